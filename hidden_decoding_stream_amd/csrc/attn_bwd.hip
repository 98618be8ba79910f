// Backward of stream-factorized attention on gfx950 (bf16 MFMA).
//
// What is computed: the gradients of the prefill attention for the loss
// sum(dO * O) (training; the page "微信WeLM提出Hidden Decoding：大模型推理新范式",
// section 实验效果与成本分析, reports the method's cost as training step
// times). With S = scale * Q K^T over the admitted keys, P = exp(S - lse),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// and under grouped-query attention a key/value head's gradients are the sums
// over its G query heads. The masks and the virtual sequences (intra: each
// stream as a strided view) are those of the forward.
//
// Three kernels, all deterministic (no atomics):
// * bwd_prep_kernel: D and lse*log2(e) per query row, into a workspace laid
//   out by virtual sequence ([B][nseq][hq][Lv][2]) so that a run of queries of
//   one virtual sequence is contiguous.
// * dK, dV (key-stationary): a wave owns 32 keys (K and V as B operands); the
//   Q and dO tiles of 64 queries stream through LDS, for each of the G query
//   heads in turn. S = Q K^T and dP = dO V^T (lane = key column), P and dS
//   with each register's own query lse / D, then dV^T += dO^T P and
//   dK^T += Q^T dS (dO^T, Q^T by transposed reads). At d = 128 every mode runs
//   bwd_dkdv128_stream_kernel, whose whole step loop is one asm stream
//   (attn_dkdv128_stream.h); d = 64 runs bwd_dkdv_kernel (three asm phases
//   per 32-query block, DkdvAsm).
// * dQ (query-stationary, shaped like the forward): per 64-key tile
//   S^T = K Q^T and dP^T = V dO^T (K and V rows from LDS as A operands, Q^T
//   and dO^T in registers), then P^T = exp2(S^T c - lse2) with the lane's own
//   lse, dS^T = P^T (dP^T - D), and dQ^T += K^T dS^T, with dS^T taken straight
//   from the accumulators as the B operand (rows read in the sigma order) and
//   K^T by transposed LDS reads. At d = 128 every mode runs bwd_dq128_kernel
//   (one wave per SIMD with 64 queries, the loop one asm stream,
//   attn_dq128_stream.h); d = 64 runs bwd_dq_kernel (two groups per CU for
//   intra and cross_full, the windowed mode one group with its loop in asm
//   phases, DqAsm).
// The d = 128 kernels keep K, V, Q and dO tiles in rows of 320 bytes whose
// 16-byte chunks are swizzled by row quad (row_swizzle128, common.h): row and
// transposed reads are then free of LDS bank conflicts. The others use rows
// padded to D+16 elements. Tiles go by buffer->LDS DMA through a ring with
// one bare barrier per tile. LDS reads are asm blocks that wait for their own
// results (see common.h), and the one-wave-per-SIMD loops run their MFMAs
// inside those blocks.
#include <math.h>

#include "attn_dkdv128_stream.h"
#include "attn_dq128_stream.h"
#include "common.h"
#include "launch.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                 // one wave per SIMD per group
constexpr int kThreads = 64 * kWaves;
constexpr int BT = 64;                    // rows per staged tile
constexpr int ST = 2;                     // LDS stages
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const u16* q;
  const u16* k;
  const u16* v;
  const u16* o;
  const u16* dout;
  const float* lse;   // [B][hq][S], natural log (from the forward)
  float* lsed;        // [B][nseq][hq][Lv][2]: lse*log2(e), D
  u16* dq;
  u16* dk;
  u16* dv;
  int32_t batch;
  int32_t S, Lv, pstride, nseq;
  int32_t hq, hkv, G, HG, hgroups;
  int32_t window;     // > 0: cross_window limit; 0: none
  float c;            // scale * log2(e)
  float scale;
  int32_t nqb, nkb;   // query blocks (dQ), key blocks (dK/dV) per virtual sequence
  int32_t total_q, per_xcd_q, total_k, per_xcd_k;
  uint32_t q_bytes, kv_bytes, lsed_bytes;
};

template <int D> struct BTile {
  static constexpr int ROW = D + 16;                       // padded row (elements)
  static constexpr int SLOTS = ROW / 8;                    // 16-byte slots per row
  static constexpr int CH = BT * SLOTS / 64;               // 1 KiB DMA chunks per tile
  static constexpr int ELEMS = BT * ROW;
  static_assert(BT * SLOTS % 64 == 0, "tile must be whole KiB chunks");
};

// 16 transposed reads gathering, for one 32-row block of a padded tile, the
// A operand X^T (rows d, k = tile rows in the accumulator order of
// reg_key_offset): output (db*2 + j2)*2 + t holds rows 16h + 4*((2t + j2) ^ h)
// + e of 32-wide d block db, from base ae (j2 = 0) or ao (j2 = 1) plus an
// immediate offset of 64 db bytes and (8t + 4j2) rows. One asm block that
// waits for its results (a builtin read would wait for every buffer->LDS load
// in flight).
template <int D> __device__ __forceinline__ void gather16(u32x2 (&x)[D / 8], uint32_t ae, uint32_t ao);
template <> __device__ __forceinline__ void gather16<64>(u32x2 (&x)[8], uint32_t ae, uint32_t ao) {
  // row offsets (8t + 4j2) * 80 elements * 2 bytes: t0j0 0, t1j0 1280, t0j1 640, t1j1 1920
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:1280\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:640\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:1920\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:1344\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:704\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:1984\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(ae), "v"(ao)
      : "memory");
}

// Two 16-wide d slices of two row operands (a from pa, b from pb, 32 bytes
// apart), in one asm block that waits only for its own results.
__device__ __forceinline__ void lds_pair2(bf16x8 (&a)[2], bf16x8 (&b)[2], uint32_t pa, uint32_t pb) {
  u32x4 x[4];
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n\t"
      "ds_read_b128 %1, %4 offset:32\n\t"
      "ds_read_b128 %2, %5 offset:0\n\t"
      "ds_read_b128 %3, %5 offset:32\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(pa), "v"(pb)
      : "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    __builtin_memcpy(&a[i], &x[i], 16);
    __builtin_memcpy(&b[i], &x[2 + i], 16);
  }
}

// Two row operands from LDS (a from pa, b from pb): 16-byte pieces at
// d = 16 kk (+ 8 hh, folded into the addresses), D / 16 of each, in one asm
// block that waits for its results, so that the compiler adds no wait for
// the buffer->LDS loads in flight.
template <int D> __device__ __forceinline__ void lds_rows2(bf16x8 (&a)[D / 16], bf16x8 (&b)[D / 16], uint32_t pa,
                                                           uint32_t pb);
template <> __device__ __forceinline__ void lds_rows2<64>(bf16x8 (&a)[4], bf16x8 (&b)[4], uint32_t pa,
                                                             uint32_t pb) {
  u32x4 x[8];
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:32\n\t"
      "ds_read_b128 %2, %8 offset:64\n\t"
      "ds_read_b128 %3, %8 offset:96\n\t"
      "ds_read_b128 %4, %9 offset:0\n\t"
      "ds_read_b128 %5, %9 offset:32\n\t"
      "ds_read_b128 %6, %9 offset:64\n\t"
      "ds_read_b128 %7, %9 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(pa), "v"(pb)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_memcpy(&a[i], &x[i], 16);
    __builtin_memcpy(&b[i], &x[4 + i], 16);
  }
}

// Per-lane pieces of the transposed-read addressing (elements, within a
// padded tile): lane i of 16-lane group grp sources tile row i/4 of its group's
// 4 rows at column 16*(grp%2) + 4*(i%4); half vh = grp/2 starts 20 rows
// further for even register groups and 12 rows for odd ones.
template <int D> struct TrBase {
  int even, odd;
  __device__ TrBase(int lane) {
    constexpr int ROW = BTile<D>::ROW;
    const int grp = lane >> 4, gi = lane & 15, vh = grp >> 1;
    const int base = (gi >> 2) * ROW + 16 * (grp & 1) + 4 * (gi & 3);
    even = base + vh * 20 * ROW;
    odd = base + vh * 12 * ROW;
  }
};

// A^T fragments of one 32-row block (starting at row r0 of the tile at LDS
// byte address tile): out[db][j2] is the A operand for the k slice whose
// B operand comes from accumulator registers 8*j2 .. 8*j2+7.
template <int D>
__device__ __forceinline__ void gather_block(bf16x8 (&out)[D / 32][2], uint32_t tile, int r0, const TrBase<D>& tb) {
  constexpr int ROW = BTile<D>::ROW;
  constexpr int DB = D / 32;
  u32x2 x[D / 8];
  gather16<D>(x, tile + uint32_t(tb.even + r0 * ROW) * 2, tile + uint32_t(tb.odd + r0 * ROW) * 2);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) __builtin_memcpy(&out[db][j2], &x[(db * 2 + j2) * 2], 16);
}

// Register operand of a 32-row block of a [.][heads][D] tensor: lane holds
// X[row0 + l32][kk*16 + 8*hh .. +8] (the B operand of a product over d, or,
// identically laid out, an A operand with rows = the 32 rows).
template <int D>
__device__ __forceinline__ void load_rows(bf16x8 (&f)[D / 16], __amdgpu_buffer_rsrc_t rs, uint32_t row_off_bytes,
                                          bool valid, int hh) {
  const uint32_t off = row_off_bytes + 16 * hh + (valid ? 0u : kOobOffset);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const uint4 x = bload16(rs, off + kk * 32);
    __builtin_memcpy(&f[kk], &x, 16);
  }
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) and lse in log2 units, per (batch, position, query head)
// ---------------------------------------------------------------------------
// One block covers kPrepRows consecutive rows of one (batch, query head) in
// the workspace's order (virtual sequence, then query), so its lse reads and
// workspace writes are contiguous; a row's O and dO are read by D/8 lanes,
// 16 bytes each, and reduced across those lanes.
constexpr int kPrepRows = 64;

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int R = D / 8;                  // lanes per row
  constexpr int SLOTS = 256 / R;            // rows per pass
  constexpr int ITER = kPrepRows / SLOTS;
  const int nblk = (p.S + kPrepRows - 1) / kPrepRows;
  const int bh = int(blockIdx.x) / nblk;    // b * hq + h
  const int j0 = (int(blockIdx.x) - bh * nblk) * kPrepRows;
  const int b = bh / p.hq, h = bh - b * p.hq;
  const int slot = int(threadIdx.x) / R, part = int(threadIdx.x) % R;
  float acc[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    acc[it] = 0.f;
    const int j = j0 + it * SLOTS + slot;   // (seq, iq) flattened: j = seq * Lv + iq
    if (j < p.S) {
      const int seq = j / p.Lv, iq = j - seq * p.Lv;
      const int pos = iq * p.pstride + seq;
      const size_t row = (size_t(b) * p.S + pos) * p.hq + h;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.o + row * D + 8 * part);
      const bf16x8 g = *reinterpret_cast<const bf16x8*>(p.dout + row * D + 8 * part);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[it] = fmaf(float(a[e]), float(g[e]), acc[it]);
    }
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
#pragma unroll
    for (int m = R / 2; m >= 1; m /= 2) acc[it] += __shfl_xor(acc[it], m, R);
    const int j = j0 + it * SLOTS + slot;
    if (j < p.S && part == 0) {
      const int seq = j / p.Lv, iq = j - seq * p.Lv;
      const int pos = iq * p.pstride + seq;
      const size_t idx = ((size_t(b) * p.nseq + seq) * p.hq + h) * p.Lv + iq;
      const float l2 = p.lse[size_t(bh) * p.S + pos] * kLog2e;
      *reinterpret_cast<float2*>(p.lsed + 2 * idx) = make_float2(l2, acc[it]);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary. Two groups share a CU (two waves per SIMD, so one
// group's waits overlap the other's work) where the registers allow it: the
// windowed mask's extra state would spill, so MODE 2 keeps one group per CU.
// ---------------------------------------------------------------------------
// The dQ loop of the windowed mode (one wave per SIMD) in three phases per
// 32-key block, each one asm block holding MFMAs and the LDS reads the next
// phase needs (the scheme of DkdvAsm below):
//   x1: S^T, dP^T over the first half of d (fresh accumulators); reads the
//       second half of the K and V rows
//   x2: the second half; gathers K^T (transposed)
//   y:  dQ^T += K^T dS^T; reads the first half of the next block's rows
template <int D> struct DqAsm;
template <> struct DqAsm<64> {
  static __device__ __forceinline__ void x1(f32x16& s, f32x16& p, const bf16x8 (&ka)[4], const bf16x8 (&va)[4],
                                            const bf16x8 (&qf)[4], const bf16x8 (&dof)[4], uint32_t pa, uint32_t pb,
                                            u32x4 (&y)[4]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[ka0], %[qf0], 0\n\t"
      "ds_read_b128 %[y0], %[pa] offset:64\n\t"
      "ds_read_b128 %[y1], %[pa] offset:96\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[va0], %[dof0], 0\n\t"
      "ds_read_b128 %[y2], %[pb] offset:64\n\t"
      "ds_read_b128 %[y3], %[pb] offset:96\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[ka1], %[qf1], %[s]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[va1], %[dof1], %[p]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [s] "=&v"(s), [p] "=&v"(p), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
      : [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [va0] "v"(va[0]), [va1] "v"(va[1]), [qf0] "v"(qf[0]),
        [qf1] "v"(qf[1]), [dof0] "v"(dof[0]), [dof1] "v"(dof[1]), [pa] "v"(pa), [pb] "v"(pb)
      : "memory");
  }
  static __device__ __forceinline__ void x2(f32x16& s, f32x16& p, const bf16x8 (&ka)[4], const bf16x8 (&va)[4],
                                            const bf16x8 (&qf)[4], const bf16x8 (&dof)[4], uint32_t ae, uint32_t ao,
                                            u32x2 (&x)[8]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[ka0], %[qf0], %[s]\n\t"
      "ds_read_b64_tr_b16 %[x0], %[ae] offset:0\n\t"
      "ds_read_b64_tr_b16 %[x1], %[ae] offset:1280\n\t"
      "ds_read_b64_tr_b16 %[x2], %[ao] offset:640\n\t"
      "ds_read_b64_tr_b16 %[x3], %[ao] offset:1920\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[va0], %[dof0], %[p]\n\t"
      "ds_read_b64_tr_b16 %[x4], %[ae] offset:64\n\t"
      "ds_read_b64_tr_b16 %[x5], %[ae] offset:1344\n\t"
      "ds_read_b64_tr_b16 %[x6], %[ao] offset:704\n\t"
      "ds_read_b64_tr_b16 %[x7], %[ao] offset:1984\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[ka1], %[qf1], %[s]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[va1], %[dof1], %[p]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 3\n\t"
      : [s] "+v"(s), [p] "+v"(p), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
        [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
      : [ka0] "v"(ka[2]), [ka1] "v"(ka[3]), [va0] "v"(va[2]), [va1] "v"(va[3]), [qf0] "v"(qf[2]),
        [qf1] "v"(qf[3]), [dof0] "v"(dof[2]), [dof1] "v"(dof[3]), [ae] "v"(ae), [ao] "v"(ao)
      : "memory");
  }
  static __device__ __forceinline__ void y(f32x16 (&acc)[2], const bf16x8 (&kT)[2][2], const bf16x8 (&dsf)[2],
                                           uint32_t pa, uint32_t pb, u32x4 (&y)[4]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t00], %[ds0], %[v0]\n\t"
      "ds_read_b128 %[y0], %[pa] offset:0\n\t"
      "ds_read_b128 %[y1], %[pa] offset:32\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t10], %[ds0], %[v1]\n\t"
      "ds_read_b128 %[y2], %[pb] offset:0\n\t"
      "ds_read_b128 %[y3], %[pb] offset:32\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t01], %[ds1], %[v0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t11], %[ds1], %[v1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [v0] "+a"(acc[0]), [v1] "+a"(acc[1]), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]),
        [y3] "=&v"(y[3])
      : [t00] "v"(kT[0][0]), [t01] "v"(kT[0][1]), [t10] "v"(kT[1][0]), [t11] "v"(kT[1][1]), [ds0] "v"(dsf[0]),
        [ds1] "v"(dsf[1]), [pa] "v"(pa), [pb] "v"(pb)
      : "memory");
  }
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, MODE == 2 ? 1 : 2) void bwd_dq_kernel(BwdParams p) {
  using TL = BTile<D>;
  constexpr int KD = D / 16, DB = D / 32;
  constexpr int NCH = 2 * TL::CH;                       // K then V chunks per tile
  constexpr int NCW = NCH / kWaves;
  static_assert(NCH % kWaves == 0, "chunks must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) u16 ks[ST][TL::ELEMS];
  __shared__ __attribute__((aligned(16))) u16 vs[ST][TL::ELEMS];

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  const int t = (blockIdx.x & 7) * p.per_xcd_q + (blockIdx.x >> 3);
  if (t >= p.total_q) return;
  const int ipu = p.nqb * p.hgroups;
  const int unit = t / ipu;
  const int rr = t - unit * ipu;
  const int qb = p.nqb - 1 - rr / p.hgroups;
  const int hg = rr % p.hgroups;
  const int kvh = unit % p.hkv;
  const int bs = unit / p.hkv;
  const int sq = bs % p.nseq;
  const int b = bs / p.nseq;
  const int h = kvh * p.G + hg * p.HG + (wave % p.HG);
  const int PS = (kWaves / p.HG) * 32;
  const int wg_q0 = qb * PS;
  const int q0 = wg_q0 + (wave / p.HG) * 32;
  const int wg_qlast = min(wg_q0 + PS, p.Lv) - 1;
  const int kt_begin = window > 0 ? max(0, wg_q0 - window + 1) / BT : 0;
  const int kt_end = wg_qlast / BT + 1;
  const int base_row = b * p.S + sq;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t dors = make_rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lsed, p.lsed_bytes);
  const uint32_t kv_pos_bytes = uint32_t(p.hkv) * D * 2;
  const uint32_t kv_head_bytes = uint32_t(kvh) * D * 2;

  // Q^T and dO^T (B operands) and the lane's query lse2 and D
  const int vq = q0 + l32;
  const bool qvalid = vq < p.Lv;
  bf16x8 qf[KD], dof[KD];
  const uint32_t qoff = (uint32_t(base_row + vq * pstride) * p.hq + h) * D * 2;
  load_rows<D>(qf, qrs, qoff, qvalid, hh);
  load_rows<D>(dof, dors, qoff, qvalid, hh);
  float lse2 = 0.f, dq_d = 0.f;
  {
    const uint32_t li = ((uint32_t(b * p.nseq + sq) * p.hq + h) * p.Lv + vq) * 8 + (qvalid ? 0u : kOobOffset);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(lrs, int(li & ~15u), 0, 0);
    const int w = (li >> 2) & 3;   // 8-byte pair within the 16 bytes
    lse2 = __uint_as_float(w == 0 ? x[0] : x[2]);
    dq_d = __uint_as_float(w == 0 ? x[1] : x[3]);
  }

  // DMA chunks: chunk c < CH is K chunk c, else V chunk c - CH; slot
  // sl = 64*chunk + lane is row sl / SLOTS, 16-byte slot sl % SLOTS (the
  // padding slots and rows past the end read zeros). The offsets are
  // recomputed per tile rather than held in registers.
  const uint32_t row_bytes = uint32_t(pstride) * kv_pos_bytes;   // between rows of a virtual sequence
  auto issue = [&](int kt) {
    const int st = kt % ST;
    const uint32_t tbase = uint32_t(base_row + kt * BT * pstride) * kv_pos_bytes + kv_head_bytes;
    // the lane's slot positions are recomputed on every call rather than held
    // in registers across the loop (the opaque copy keeps the compiler from
    // hoisting them)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const int c = wave + j * kWaves;
      const int sl = (c < TL::CH ? c : c - TL::CH) * 64 + ln;
      const int row = sl / TL::SLOTS, ch = sl % TL::SLOTS;
      const bool ok = ch < D / 8 && kt * BT + row < p.Lv;
      const uint32_t off = ok ? tbase + uint32_t(row) * row_bytes + ch * 16 : kOobOffset;
      if (c < TL::CH) dma16(krs, &ks[st][c * 512], off);
      else dma16(vrs, &vs[st][(c - TL::CH) * 512], off);
    }
  };

  const int rowA = sigma(l32);               // tile row (within a 32-row block) this lane reads as A
  const TrBase<D> tb(lane);
  const int qhi = min(q0 + 32, p.Lv) - 1;
  const bool wave_live = q0 < p.Lv;
  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  issue(kt_begin);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");
  if constexpr (MODE == 2) {
    // one wave per SIMD: the phases in asm (DqAsm), every tile processed and
    // masked (no per-wave skip, so that the prefetch chain stays unbroken)
    constexpr int H = KD / 2;
    constexpr uint32_t kStageBytes = TL::ELEMS * 2;
    const uint32_t ks0 = lds_addr(&ks[0][0]), vs0 = lds_addr(&vs[0][0]);
    auto rows_at = [&](uint32_t base, int st, int kb) {
      return base + st * kStageBytes + uint32_t((kb * 32 + rowA) * TL::ROW + 8 * hh) * 2;
    };
    const uint32_t lim = uint32_t(window);
    bf16x8 ka[KD], va[KD];
    lds_rows2<D>(ka, va, rows_at(ks0, kt_begin % ST, 0), rows_at(vs0, kt_begin % ST, 0));
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int st = kt % ST;
      const int k0 = kt * BT;
      if (kt + 1 < kt_end) issue(kt + 1);
      const bool full = (k0 + BT - 1 <= q0) && (window == 0 || qhi - k0 < window);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc, pacc;
        {
          u32x4 y[KD];
          DqAsm<D>::x1(sacc, pacc, ka, va, qf, dof, rows_at(ks0, st, kb), rows_at(vs0, st, kb), y);
#pragma unroll
          for (int k = 0; k < H; ++k) {
            __builtin_memcpy(&ka[H + k], &y[k], 16);
            __builtin_memcpy(&va[H + k], &y[H + k], 16);
          }
        }
        bf16x8 kT[DB][2];
        {
          u32x2 x[D / 8];
          const uint32_t tile = ks0 + st * kStageBytes;
          const uint32_t ae = tile + uint32_t(tb.even + kb * 32 * TL::ROW) * 2;
          const uint32_t ao = tile + uint32_t(tb.odd + kb * 32 * TL::ROW) * 2;
          DqAsm<D>::x2(sacc, pacc, ka, va, qf, dof, ae, ao, x);
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) __builtin_memcpy(&kT[db][j2], &x[(db * 2 + j2) * 2], 16);
        }
        bf16x8 dsf[2];
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int reg = j2 * 8 + i;
            float s = sacc[reg];
            if (!full) {
              const int key = k0 + kb * 32 + reg_key_offset(reg >> 2, hh) + (reg & 3);
              if (!(uint32_t(vq - key) < lim)) s = -INFINITY;
            }
            const float pr = __builtin_amdgcn_exp2f(fmaf(s, p.c, -lse2));
            dsf[j2][i] = (__bf16)(pr * (pacc[reg] - dq_d));
          }
        }
        // the next block's rows: (kt, 1) from this stage, or (kt + 1, 0) from
        // the next one once it is published (after the last tile a harmless
        // read of a stage no DMA writes)
        int nst = st, nkb = 1;
        if (kb == 1) {
          if (kt + 1 < kt_end) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");   // every read of this stage has returned above
          }
          nst = (kt + 1) % ST;
          nkb = 0;
        }
        {
          u32x4 y[KD];
          DqAsm<D>::y(dqacc, kT, dsf, rows_at(ks0, nst, nkb), rows_at(vs0, nst, nkb), y);
#pragma unroll
          for (int k = 0; k < H; ++k) {
            __builtin_memcpy(&ka[k], &y[k], 16);
            __builtin_memcpy(&va[k], &y[H + k], 16);
          }
        }
      }
    }
    // accumulators written by MFMAs are read by the epilogue below
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  } else {
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int st = kt % ST;
      const int k0 = kt * BT;
      if (kt + 1 < kt_end) issue(kt + 1);
      const bool live = wave_live && k0 <= qhi && !(window > 0 && q0 - (k0 + BT - 1) >= window);
      if (live) {
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // K and V rows, two 16-wide d slices at a time, by asm reads that wait
          // only for themselves (a C++ read here made the compiler wait for the
          // next tile's DMA first)
          const uint32_t pk = lds_addr(&ks[st][(kb * 32 + rowA) * TL::ROW + 8 * hh]);
          const uint32_t pv = lds_addr(&vs[st][(kb * 32 + rowA) * TL::ROW + 8 * hh]);
          sacc[kb] = f32x16{};
          pacc[kb] = f32x16{};
#pragma unroll
          for (int j = 0; j < KD / 2; ++j) {
            bf16x8 ka[2], va[2];
            lds_pair2(ka, va, pk + 64 * j, pv + 64 * j);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t], qf[2 * j + t], sacc[kb], 0, 0, 0);
              pacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], dof[2 * j + t], pacc[kb], 0, 0, 0);
            }
          }
        }
        // K^T fragments for dQ^T += K^T dS^T
        bf16x8 kT[2][DB][2];
        const uint32_t kt_lds = lds_addr(&ks[st][0]);
        gather_block<D>(kT[0], kt_lds, 0, tb);
        gather_block<D>(kT[1], kt_lds, 32, tb);

        const bool full = (k0 + BT - 1 <= q0) && (window == 0 || qhi - k0 < window);
        const uint32_t lim = MODE == 2 ? uint32_t(window) : 0x80000000u;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 dsf[2];
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int reg = j2 * 8 + i;
              float s = sacc[kb][reg];
              if (!full) {
                const int key = k0 + kb * 32 + reg_key_offset(reg >> 2, hh) + (reg & 3);
                if (!(uint32_t(vq - key) < lim)) s = -INFINITY;
              }
              const float pr = __builtin_amdgcn_exp2f(fmaf(s, p.c, -lse2));
              dsf[j2][i] = (__bf16)(pr * (pacc[kb][reg] - dq_d));
            }
          }
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2)
              dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT[kb][db][j2], dsf[j2], dqacc[db], 0, 0, 0);
        }
      }
      if (kt + 1 < kt_end) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");   // no fence needed: every read of stage st was consumed above
      }
    }
  }

  if (!qvalid) return;
  u16* orow = p.dq + (size_t(base_row + vq * pstride) * p.hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 ov;
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(dqacc[db][4 * g + r] * p.scale);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hh) = ov;
    }
}


// The d = 64 dK/dV loop in three phases per 32-query block, each one asm block that
// issues the phase's MFMAs with the LDS reads the next phase needs spread over
// the first half of them, and waits for those reads only at its end: with one
// wave per SIMD, nothing else would keep the matrix core busy while a read is
// outstanding. The MFMAs sit in the same block as the reads because a read
// left in flight across asm blocks could land in a register the compiler has
// meanwhile reused. Wait states the compiler cannot see inside asm are
// explicit: s_nop 2 before MFMAs that read VALU-written registers, and 20
// after the score MFMAs whose results the VALU reads next.
//   x:  S = Q K^T, dP = dO V^T (fresh accumulators); reads dO^T (transposed)
//       and the block's (lse2, D) pairs
//   y1: dV^T += dO^T P; reads Q^T (transposed)
//   y2: dK^T += Q^T dS; reads the next block's Q and dO rows
// Same products in the same accumulation order as builtin MFMAs would give.
template <int D> struct DkdvAsm;
template <> struct DkdvAsm<64> {
  // S = Q K^T and dP = dO V^T (fresh accumulators), with dO^T gathered and the
  // block's (lse2, D) pairs read
  static __device__ __forceinline__ void x(f32x16& s, f32x16& p, const bf16x8 (&qa)[4], const bf16x8 (&da)[4],
                                           const bf16x8 (&kf)[4], const bf16x8 (&vf)[4], uint32_t ae, uint32_t ao,
                                           const uint32_t (&r)[4], u32x2 (&x)[8], u32x4 (&y)[8]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[qa0], %[kf0], 0\n\t"
      "ds_read_b64_tr_b16 %[x0], %[ae] offset:0\n\t"
      "ds_read_b64_tr_b16 %[x1], %[ae] offset:1280\n\t"
      "ds_read_b64_tr_b16 %[x2], %[ao] offset:640\n\t"
      "ds_read_b64_tr_b16 %[x3], %[ao] offset:1920\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[da0], %[vf0], 0\n\t"
      "ds_read_b64_tr_b16 %[x4], %[ae] offset:64\n\t"
      "ds_read_b64_tr_b16 %[x5], %[ae] offset:1344\n\t"
      "ds_read_b64_tr_b16 %[x6], %[ao] offset:704\n\t"
      "ds_read_b64_tr_b16 %[x7], %[ao] offset:1984\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[qa1], %[kf1], %[s]\n\t"
      "ds_read_b128 %[y0], %[r0] offset:0\n\t"
      "ds_read_b128 %[y1], %[r0] offset:16\n\t"
      "ds_read_b128 %[y2], %[r1] offset:0\n\t"
      "ds_read_b128 %[y3], %[r1] offset:16\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[da1], %[vf1], %[p]\n\t"
      "ds_read_b128 %[y4], %[r2] offset:0\n\t"
      "ds_read_b128 %[y5], %[r2] offset:16\n\t"
      "ds_read_b128 %[y6], %[r3] offset:0\n\t"
      "ds_read_b128 %[y7], %[r3] offset:16\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[qa2], %[kf2], %[s]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[da2], %[vf2], %[p]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[s], %[qa3], %[kf3], %[s]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[p], %[da3], %[vf3], %[p]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 3\n\t"
      : [s] "=&v"(s), [p] "=&v"(p), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
        [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7]), [y0] "=&v"(y[0]),
        [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3]), [y4] "=&v"(y[4]), [y5] "=&v"(y[5]),
        [y6] "=&v"(y[6]), [y7] "=&v"(y[7])
      : [qa0] "v"(qa[0]), [qa1] "v"(qa[1]), [qa2] "v"(qa[2]), [qa3] "v"(qa[3]), [da0] "v"(da[0]),
        [da1] "v"(da[1]), [da2] "v"(da[2]), [da3] "v"(da[3]), [kf0] "v"(kf[0]), [kf1] "v"(kf[1]),
        [kf2] "v"(kf[2]), [kf3] "v"(kf[3]), [vf0] "v"(vf[0]), [vf1] "v"(vf[1]), [vf2] "v"(vf[2]),
        [vf3] "v"(vf[3]), [ae] "v"(ae), [ao] "v"(ao), [r0] "v"(r[0]), [r1] "v"(r[1]), [r2] "v"(r[2]),
        [r3] "v"(r[3])
      : "memory");
  }
  // acc[db] += opA[db][j] opB[j] (dV^T += dO^T P), with Q^T gathered
  static __device__ __forceinline__ void y1(f32x16 (&acc)[2], const bf16x8 (&opA)[2][2], const bf16x8 (&opB)[2],
                                            uint32_t ae, uint32_t ao, u32x2 (&x)[8]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t00], %[pf0], %[v0]\n\t"
      "ds_read_b64_tr_b16 %[x0], %[ae] offset:0\n\t"
      "ds_read_b64_tr_b16 %[x1], %[ae] offset:1280\n\t"
      "ds_read_b64_tr_b16 %[x2], %[ao] offset:640\n\t"
      "ds_read_b64_tr_b16 %[x3], %[ao] offset:1920\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t10], %[pf0], %[v1]\n\t"
      "ds_read_b64_tr_b16 %[x4], %[ae] offset:64\n\t"
      "ds_read_b64_tr_b16 %[x5], %[ae] offset:1344\n\t"
      "ds_read_b64_tr_b16 %[x6], %[ao] offset:704\n\t"
      "ds_read_b64_tr_b16 %[x7], %[ao] offset:1984\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t01], %[pf1], %[v0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t11], %[pf1], %[v1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [v0] "+a"(acc[0]), [v1] "+a"(acc[1]), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]),
        [x3] "=&v"(x[3]), [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
      : [t00] "v"(opA[0][0]), [t01] "v"(opA[0][1]), [t10] "v"(opA[1][0]), [t11] "v"(opA[1][1]),
        [pf0] "v"(opB[0]), [pf1] "v"(opB[1]), [ae] "v"(ae), [ao] "v"(ao)
      : "memory");
  }
  // acc[db] += opA[db][j] opB[j] (dK^T += Q^T dS), with the next block's Q and dO rows read
  static __device__ __forceinline__ void y2(f32x16 (&acc)[2], const bf16x8 (&opA)[2][2], const bf16x8 (&opB)[2],
                                            uint32_t pa, uint32_t pb, u32x4 (&y)[8]) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t00], %[pf0], %[v0]\n\t"
      "ds_read_b128 %[y0], %[pa] offset:0\n\t"
      "ds_read_b128 %[y1], %[pa] offset:32\n\t"
      "ds_read_b128 %[y2], %[pa] offset:64\n\t"
      "ds_read_b128 %[y3], %[pa] offset:96\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t10], %[pf0], %[v1]\n\t"
      "ds_read_b128 %[y4], %[pb] offset:0\n\t"
      "ds_read_b128 %[y5], %[pb] offset:32\n\t"
      "ds_read_b128 %[y6], %[pb] offset:64\n\t"
      "ds_read_b128 %[y7], %[pb] offset:96\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v0], %[t01], %[pf1], %[v0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[v1], %[t11], %[pf1], %[v1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [v0] "+a"(acc[0]), [v1] "+a"(acc[1]), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]),
        [y3] "=&v"(y[3]), [y4] "=&v"(y[4]), [y5] "=&v"(y[5]), [y6] "=&v"(y[6]), [y7] "=&v"(y[7])
      : [t00] "v"(opA[0][0]), [t01] "v"(opA[0][1]), [t10] "v"(opA[1][0]), [t11] "v"(opA[1][1]),
        [pf0] "v"(opB[0]), [pf1] "v"(opB[1]), [pa] "v"(pa), [pb] "v"(pb)
      : "memory");
  }
};

// ---------------------------------------------------------------------------
// The d = 128 tile layout (Q / dO tiles of the dK/dV kernel, K / V tiles of
// the dQ kernel)
// ---------------------------------------------------------------------------
// gfx950 LDS has 64 banks of 4 bytes. A 16-byte read (ds_read_b128) is served
// in four passes of 16 lanes: within each half-wave, the lanes whose quad
// index (lane / 4 mod 8) has the same parity. 8-byte reads (ds_read_b64 and
// the transposed ds_read_b64_tr_b16) are served in two passes of 32 lanes.
// A pass in which no two lanes hit one bank at different addresses takes one
// cycle. With rows padded to D+16 elements every row read and every
// transposed read of these tiles met two lanes per bank; this layout meets
// none:
// * row r holds its 128 bf16 as 16 chunks of 16 bytes at r * 320
//   bytes, chunk c in slot c ^ s(r) with s(r) = (q & 3) ^ ((q >> 2) & 1) for
//   the row quad q = r / 4; slots 16-19 stay unused (the DMA moves zeros).
// * transposed reads: a pass reads 64 contiguous bytes (chunks 4 db .. 4 db
//   + 3) of each row of one aligned row quad; the rows start 64 bytes apart
//   modulo 256, and the XOR only permutes chunks inside those 64 bytes.
// * row reads (MFMA A operands, sigma order): a pass reads chunk c of 4 rows
//   from each of 4 row quads; the rows of a quad lie 64 bytes apart modulo
//   256, and the 4 quads of a pass (sigma groups {0,7,4,3} or {5,2,1,6},
//   plus 8 for the second 32 rows) have distinct s, which moves them to
//   distinct 16-byte slots inside those 64 bytes.
// Only the two low bits of the chunk index change, so a lane's transposed
// reads sit at immediate offsets 64 db from one base per row offset, and its
// row reads at 64 j from one base for the even and one for the odd k-steps.
constexpr int kRowBytes128 = 320;
constexpr int kTileBytes128 = 64 * kRowBytes128;

// ---------------------------------------------------------------------------
// dK, dV: key-stationary
// ---------------------------------------------------------------------------
template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  using TL = BTile<D>;
  constexpr int KD = D / 16, DB = D / 32;
  constexpr int NCH = 2 * TL::CH;                       // Q then dO chunks per tile
  constexpr int NCW = NCH / kWaves;                     // chunks per wave (wave 0 also moves lse2/D)
  static_assert(NCH % kWaves == 0, "chunks must split evenly over the waves");
  constexpr int KB = kWaves * 32;                       // keys per work group
  constexpr int SK = 3;                                 // LDS stages: step s + 2 loads while s runs
  __shared__ __attribute__((aligned(16))) u16 qs[SK][TL::ELEMS];
  __shared__ __attribute__((aligned(16))) u16 ds_[SK][TL::ELEMS];
  __shared__ __attribute__((aligned(16))) float ls[SK][2 * 64 * 2];   // [query][lse2, D], 1 KiB per stage

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // work item: (batch, virtual sequence, kv head, key block), heaviest first
  const int t = (blockIdx.x & 7) * p.per_xcd_k + (blockIdx.x >> 3);
  if (t >= p.total_k) return;
  const int unit = t / p.nkb;
  const int kbk = t - unit * p.nkb;          // key block 0 has the most queries above it
  const int kvh = unit % p.hkv;
  const int bs = unit / p.hkv;
  const int sq = bs % p.nseq;
  const int b = bs / p.nseq;
  const int base_row = b * p.S + sq;
  const int wg_k0 = kbk * KB;
  const int k0 = wg_k0 + wave * 32;
  const int vk = k0 + l32;                    // this lane's key (virtual index)
  const bool kvalid = vk < p.Lv;
  const int wg_klast = min(wg_k0 + KB, p.Lv) - 1;
  // query tiles that can see a key of the block: from the block's first key
  // to its last key plus the window
  const int qt_begin = wg_k0 / BT;
  const int qlast = window > 0 ? min(p.Lv - 1, wg_klast + window - 1) : p.Lv - 1;
  const int qt_end = qlast / BT + 1;
  const int nsteps = (qt_end - qt_begin) * p.G;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t dors = make_rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lsed, p.lsed_bytes);
  const uint32_t q_pos_bytes = uint32_t(p.hq) * D * 2;
  const uint32_t lbase_seq = uint32_t(b * p.nseq + sq) * p.hq;   // workspace row of head 0 (times Lv)

  // K and V of this lane's key as B operands (K^T, V^T: k = d, n = key)
  bf16x8 kf[KD], vf[KD];
  {
    const uint32_t koff = (uint32_t(base_row + vk * pstride) * p.hkv + kvh) * D * 2;
    load_rows<D>(kf, krs, koff, kvalid, hh);
    load_rows<D>(vf, vrs, koff, kvalid, hh);
  }

  // step s: query tile qt_begin + s / G, query head kvh*G + s % G. Chunk c
  // of a tile (c < CH: Q, else dO) puts slot sl = 64 (c mod CH) + lane at
  // row sl / SLOTS, 16-byte slot sl % SLOTS (the padding slots read zeros);
  // wave w moves chunks w, w + 4, ...; wave 0 also moves the 64 queries'
  // (lse2, D) pairs, 16 bytes per lane.
  auto issue = [&](int s) {
    const int st = s % SK;
    const int qt = qt_begin + s / p.G;
    const int h = kvh * p.G + s % p.G;
    const uint32_t tbase = uint32_t(base_row + qt * BT * pstride) * q_pos_bytes + uint32_t(h) * D * 2;
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const int c = wave + j * kWaves;
      const int sl = (c < TL::CH ? c : c - TL::CH) * 64 + lane;
      const int row = sl / TL::SLOTS, ch = sl % TL::SLOTS;
      const bool ok = ch < D / 8 && qt * BT + row < p.Lv;
      const uint32_t off = ok ? tbase + uint32_t(row * pstride) * q_pos_bytes + ch * 16 : kOobOffset;
      if (c < TL::CH) dma16(qrs, &qs[st][c * 512], off);
      else dma16(dors, &ds_[st][(c - TL::CH) * 512], off);
    }
    if (wave == 0) {
      const int iq = qt * BT + 2 * lane;
      const uint32_t off = lane < 32 && iq < p.Lv ? ((lbase_seq + h) * p.Lv + iq) * 8 : kOobOffset;
      dma16(lrs, &ls[st][0], off);
    }
  };
  // this wave's chunks of the latest issued step may stay in flight
  auto wait_prev = [&](bool keep) {
    if (!keep) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (wave == 0) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCW + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCW) : "memory");
  };

  const int rowA = sigma(l32);
  const TrBase<D> tb(lane);
  const uint32_t lim = MODE == 2 ? uint32_t(window) : 0x80000000u;
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  if (nsteps > 0) {
    issue(0);
    if (nsteps > 1) issue(1);
    wait_prev(nsteps > 1);
    asm volatile("s_barrier" ::: "memory");
  }
  constexpr uint32_t kStageBytes = TL::ELEMS * 2, kLsBytes = 2 * 64 * 2 * 4;
  const uint32_t qs0 = lds_addr(&qs[0][0]), ds0 = lds_addr(&ds_[0][0]), ls0 = lds_addr(&ls[0][0]);
  auto rows_at = [&](uint32_t base, int st, int qb) {
    return base + st * kStageBytes + uint32_t((qb * 32 + rowA) * TL::ROW + 8 * hh) * 2;
  };
  bf16x8 qa[KD], da[KD];
  if (nsteps > 0) lds_rows2<D>(qa, da, rows_at(qs0, 0, 0), rows_at(ds0, 0, 0));
  for (int s = 0; s < nsteps; ++s) {
    const int st = s % SK;
    const int qt = qt_begin + s / p.G;
    // stage (s + 2) % 3 held step s - 1, which every wave has finished
    if (s + 2 < nsteps) issue(s + 2);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qf0 = qt * BT + qb * 32;        // first query of the block
      // the block is full when every query sees every key of the wave and all queries are valid
      const bool full = qf0 + 31 < p.Lv && k0 + 31 <= qf0 && (window == 0 || qf0 + 31 - k0 < window);
      f32x16 sacc, pacc;
      bf16x8 doT[DB][2];
      float l2[16], dd[16];
      {
        u32x2 x[D / 8];
        u32x4 y[8];
        const uint32_t tile = ds0 + st * kStageBytes;
        const uint32_t ae = tile + uint32_t(tb.even + qb * 32 * TL::ROW) * 2;
        const uint32_t ao = tile + uint32_t(tb.odd + qb * 32 * TL::ROW) * 2;
        uint32_t r[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) r[g] = ls0 + st * kLsBytes + 8 * (qb * 32 + reg_key_offset(g, hh));
        DkdvAsm<D>::x(sacc, pacc, qa, da, kf, vf, ae, ao, r, x, y);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2) __builtin_memcpy(&doT[db][j2], &x[(db * 2 + j2) * 2], 16);
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4& v = y[2 * g + e / 2];
            l2[4 * g + e] = __uint_as_float(v[2 * (e & 1)]);
            dd[4 * g + e] = __uint_as_float(v[2 * (e & 1) + 1]);
          }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int reg = j2 * 8 + i;
          float sc = sacc[reg];
          if (!full) {
            const int iq = qf0 + reg_key_offset(reg >> 2, hh) + (reg & 3);
            if (!(iq < p.Lv && uint32_t(iq - vk) < lim)) sc = -INFINITY;
          }
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc, p.c, -l2[reg]));
          pf[j2][i] = (__bf16)pr;
          dsf[j2][i] = (__bf16)(pr * (pacc[reg] - dd[reg]));
        }
      bf16x8 qT[DB][2];
      {
        u32x2 x[D / 8];
        const uint32_t tile = qs0 + st * kStageBytes;
        const uint32_t ae = tile + uint32_t(tb.even + qb * 32 * TL::ROW) * 2;
        const uint32_t ao = tile + uint32_t(tb.odd + qb * 32 * TL::ROW) * 2;
        DkdvAsm<D>::y1(dvacc, doT, pf, ae, ao, x);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2) __builtin_memcpy(&qT[db][j2], &x[(db * 2 + j2) * 2], 16);
      }
      // the next block's rows: (s, 1) from this stage, or (s + 1, 0) from the
      // next one once it is published (on the last step a harmless read of a
      // stage no DMA writes)
      int nst = st, nqb = 1;
      if (qb == 1) {
        if (s + 1 < nsteps) {
          // step s + 1 must have landed; the chunks of step s + 2 may still fly
          wait_prev(s + 2 < nsteps);
          asm volatile("s_barrier" ::: "memory");   // every read of this stage has returned above
        }
        nst = (s + 1) % SK;
        nqb = 0;
      }
      {
        u32x4 y[2 * KD];
        DkdvAsm<D>::y2(dkacc, qT, dsf, rows_at(qs0, nst, nqb), rows_at(ds0, nst, nqb), y);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          __builtin_memcpy(&qa[kk], &y[kk], 16);
          __builtin_memcpy(&da[kk], &y[KD + kk], 16);
        }
      }
    }
  }
  // accumulators written by MFMAs are read by the epilogue below
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");

  if (!kvalid) return;
  const size_t krow = (size_t(base_row + vk * pstride) * p.hkv + kvh) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 kv, vv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kv[r] = (__bf16)(dkacc[db][4 * g + r] * p.scale);
        vv[r] = (__bf16)dvacc[db][4 * g + r];
      }
      *reinterpret_cast<bf16x4*>(p.dk + krow + db * 32 + 8 * g + 4 * hh) = kv;
      *reinterpret_cast<bf16x4*>(p.dv + krow + db * 32 + 8 * g + 4 * hh) = vv;
    }
}

// ---------------------------------------------------------------------------
// dK, dV at d = 128: the work items and products of bwd_dkdv_kernel in the
// 320-byte tile layout, with the whole step loop as one asm stream
// (attn_dkdv128_stream.h, written by gen_dkdv128_stream.py), so that no
// compiled code runs between blocks: the DMA offsets advance by per-step
// increments, and the (lse2, D) pairs of a step come by DMA too (each wave
// moves 16 queries' pairs, into a KiB of its own). Masks: the query tiles
// whose every query sees every key of the wave form one range per wave,
// tested with two scalar instructions; the other steps (the diagonal, the
// window's end, a ragged last tile, and the step after the last, which
// closes the stream) test each score against its query and the lane's key.
// The query tiles are walked from the last down, so that the work groups of
// an XCD, which start together, read the same Q and dO tiles at about the
// same time (from L2). Rows past the end of a sequence load the next rows of
// the buffer (or zeros past its end), which the masks exclude.
// ---------------------------------------------------------------------------
constexpr int kKvTile = 20480;                 // bytes of a Q (or dO) tile
constexpr int kKvDRegion = 3 * kKvTile;        // the 3 dO tiles follow the 3 Q tiles
constexpr int kKvLRegion = 6 * kKvTile;        // then the pairs, 4 KiB per stage
constexpr int kKvLStage = 4096;

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv128_stream_kernel(BwdParams p) {
  constexpr int D = 128;
  constexpr int KB = kWaves * 32;                      // keys per work group
  static_assert(kKvTile == kTileBytes128, "the stream's offsets assume 20480-byte tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kKvLRegion + 3 * kKvLStage];

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // work item: (batch, virtual sequence, kv head, key block), heaviest first
  const int t = (blockIdx.x & 7) * p.per_xcd_k + (blockIdx.x >> 3);
  if (t >= p.total_k) return;
  const int unit = t / p.nkb;
  const int kbk = t - unit * p.nkb;
  const int kvh = unit % p.hkv;
  const int bs = unit / p.hkv;
  const int sq = bs % p.nseq;
  const int b = bs / p.nseq;
  const int base_row = b * p.S + sq;
  const int wg_k0 = kbk * KB;
  const int k0 = wg_k0 + wave * 32;
  const int vk = k0 + l32;
  const bool kvalid = vk < p.Lv;
  const int qt_begin = wg_k0 / BT;
  const int64_t W = window > 0 ? window : 0x7fffffff;
  const int qt_end = int(min<int64_t>(p.Lv - 1, int64_t(min(wg_k0 + KB, p.Lv) - 1) + W - 1) / BT) + 1;
  const int G = p.G;
  const int T = (qt_end - qt_begin) * G;               // steps: (query tile, head of the group)

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t dors = make_rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lsed, p.lsed_bytes);
  const uint32_t q_pos_bytes = uint32_t(p.hq) * D * 2;
  const uint32_t lbase_seq = uint32_t(b * p.nseq + sq) * p.hq;

  // K^T and V^T (B operands: lane holds row vk, d = 16 kk + 8 hh .. + 8)
  typedef __bf16 bf16x64 __attribute__((ext_vector_type(64)));
  bf16x64 kf, vf;
  {
    const uint32_t off = (uint32_t(base_row + vk * pstride) * p.hkv + kvh) * D * 2 + 16 * hh +
                         (kvalid ? 0u : kOobOffset);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 x = bload16(krs, off + kk * 32);
      __builtin_memcpy(reinterpret_cast<char*>(&kf) + kk * 16, &x, 16);
      const uint4 y = bload16(vrs, off + kk * 32);
      __builtin_memcpy(reinterpret_cast<char*>(&vf) + kk * 16, &y, 16);
    }
  }

  // DMA chunks of this wave: chunk w + 4 x (x < 5) of the Q tile and the same
  // chunk of the dO tile (slot sl = 64 chunk + lane is 16-byte slot u = sl mod 20
  // of row sl / 20, holding data chunk u ^ row_swizzle128(row / 4); slots 16-19
  // padding), and the pairs of queries 16 w .. 16 w + 15 (lanes 0-7, 16 bytes each)
  uint32_t cf[5];
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const int sl = (wave + 4 * x) * 64 + lane;
    const int row = sl / 20, u = sl % 20;
    cf[x] = u >= 16 ? kOobOffset : uint32_t(row * pstride) * q_pos_bytes + (u ^ row_swizzle128(row >> 2)) * 16;
  }
  auto step_base = [&](int s) {
    const int qt = qt_end - 1 - s / G, h = kvh * G + s % G;
    return uint32_t(base_row + qt * BT * pstride) * q_pos_bytes + uint32_t(h) * D * 2;
  };
  auto pair_off = [&](int s) {
    const int qt = qt_end - 1 - s / G, h = kvh * G + s % G;
    return lane < 8 && s < T ? ((lbase_seq + h) * uint32_t(p.Lv) + uint32_t(qt * BT + 16 * wave + 2 * lane)) * 8
                             : kOobOffset;
  };
  auto chunk = [&](int x, int s) { return (s < T && cf[x] < kOobOffset) ? cf[x] + step_base(s) : kOobOffset; };
  // step 0 into stage 0, zeros into the Q and dO tiles of stage 2 (the first
  // step's transposed reads of a step -1, whose P and dS are 0), step 1 into stage 1
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    dma16(qrs, &lds[(wave + 4 * x) * 1024], chunk(x, 0));
    dma16(dors, &lds[kKvDRegion + (wave + 4 * x) * 1024], chunk(x, 0));
  }
  dma16(lrs, &lds[kKvLRegion + wave * 1024], pair_off(0));
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    dma16(qrs, &lds[2 * kKvTile + (wave + 4 * x) * 1024], kOobOffset);
    dma16(dors, &lds[kKvDRegion + 2 * kKvTile + (wave + 4 * x) * 1024], kOobOffset);
  }
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    dma16(qrs, &lds[kKvTile + (wave + 4 * x) * 1024], chunk(x, 1));
    dma16(dors, &lds[kKvDRegion + kKvTile + (wave + 4 * x) * 1024], chunk(x, 1));
  }
  dma16(lrs, &lds[kKvLRegion + kKvLStage + wave * 1024], pair_off(1));
  // the loop's first DMA is step 2
#pragma unroll
  for (int x = 0; x < 5; ++x) cf[x] = chunk(x, 2);
  uint32_t cl = pair_off(2);

  // LDS read bases (stages, blocks and d slices at immediate offsets): rows of
  // a 32-row block in the sigma order (even k-steps from qe, odd from qo; dO
  // from ge / go), transposed reads for (t, jj) from q<t><jj> / d<t><jj>, and
  // the pairs of registers 0-7 / 8-15 from lp0 / lp1 (the lane half's KiB)
  const uint32_t lds0 = lds_addr(&lds[0]);
  uint32_t qe, qo;
  {
    const int r = sigma(l32), sw = row_swizzle128(r >> 2);
    const uint32_t rb = lds0 + uint32_t(r * kRowBytes128 + 16 * (hh ^ (sw & 1)));
    qe = rb + 32 * (sw >> 1);
    qo = rb + 32 - 32 * (sw >> 1);
  }
  uint32_t tq[4];
  {
    const int grp = lane >> 4, gi = lane & 15, vh = grp >> 1, e = gi >> 2;
    const int c0 = 2 * (grp & 1) + ((gi & 3) >> 1), half = gi & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = i & 1, jj = i >> 1;
      const int ro = jj ? 12 * vh + 4 + 8 * tt : 20 * vh + 8 * tt;
      tq[i] = lds0 + uint32_t((e + ro) * kRowBytes128 + 16 * (c0 ^ row_swizzle128(ro >> 2)) + 8 * half);
    }
  }
  const uint32_t lpb = lds0 + kKvLRegion + uint32_t(hh) * 1024;
  const uint32_t lp0 = lpb + 8 * uint32_t(reg_key_offset(0, hh) - 16 * hh);
  const uint32_t lp1 = lpb + 8 * uint32_t(reg_key_offset(2, hh) - 16 * hh);

  // masks: the query tiles whose every query (valid, and within the window)
  // sees every key of the wave (qt*64 >= k0 + 31, qt*64 + 63 - k0 < W,
  // qt*64 + 63 < Lv), as processed indices fd .. fd + fc - 1; the other steps
  // test each score (lane key vk, query offsets by register group in off)
  auto fdiv64 = [](int64_t x) { return x >= 0 ? x / BT : -((-x + BT - 1) / BT); };   // floor(x / 64)
  const int64_t fa = max<int64_t>(qt_begin, (int64_t(k0) + 31 + BT - 1) / BT);
  const int64_t fb = min<int64_t>(qt_end - 1, min(fdiv64(int64_t(k0) + W - BT), fdiv64(int64_t(p.Lv) - BT)));
  const uint32_t fd = __builtin_amdgcn_readfirstlane(uint32_t(qt_end - 1 - fb));
  const uint32_t fc = __builtin_amdgcn_readfirstlane(uint32_t(max<int64_t>(0, fb - fa + 1)));
  const uint32_t qtop = __builtin_amdgcn_readfirstlane(uint32_t((qt_end - 1) * BT));
  const uint32_t Wn = uint32_t(W), Lvn = uint32_t(p.Lv);
  uint32_t off = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) off |= uint32_t(reg_key_offset(g, hh)) << (8 * g);

  const uint32_t lw = __builtin_amdgcn_readfirstlane(lds0 + uint32_t(wave) * 1024);
  const uint32_t Tn = __builtin_amdgcn_readfirstlane(uint32_t(T));
  const uint32_t Gn = uint32_t(G);
  // offset steps (mod 2^32): next head, or the tile below and the first head
  const uint32_t incw = 0u - uint32_t(BT * pstride) * q_pos_bytes - uint32_t(G - 1) * D * 2;
  const uint32_t inclh = uint32_t(p.Lv) * 8, inclw = 0u - uint32_t(BT) * 8 - uint32_t(G - 1) * uint32_t(p.Lv) * 8;

  // step 0 and the zeros landed for every wave (step 1 may still be in flight)
  asm volatile("s_waitcnt vmcnt(11)\n\ts_barrier" ::: "memory");

  typedef float f32x32 __attribute__((ext_vector_type(32)));
  f32x32 dka, dkb, dva, dvb;
  asm volatile(
      SFA_DKDV128_PROLOGUE
      SFA_DKDV128_LOOP
      "s_waitcnt lgkmcnt(0)\n"
      "s_nop 7\n"
      "s_nop 7\n"
      : [dka] "={a[0:31]}"(dka), [dkb] "={a[32:63]}"(dkb), [dva] "={a[64:95]}"(dva), [dvb] "={a[96:127]}"(dvb),
        [cf0] "+v"(cf[0]), [cf1] "+v"(cf[1]), [cf2] "+v"(cf[2]), [cf3] "+v"(cf[3]), [cf4] "+v"(cf[4]),
        [cl] "+v"(cl)
      : [kf] "{a[128:159]}"(kf), [vf] "{a[160:191]}"(vf), [c] "s"(p.c), [T] "s"(Tn), [G] "s"(Gn),
        [fd] "s"(fd), [fc] "s"(fc), [qtop] "s"(qtop), [W] "s"(Wn), [Lv] "s"(Lvn), [incw] "s"(incw), [inclw] "s"(inclw), [inclh] "s"(inclh),
        [rq] "s"(qrs), [rd] "s"(dors), [rl] "s"(lrs), [lw] "s"(lw),
        [qe] "v"(qe), [qo] "v"(qo), [ge] "v"(qe + kKvDRegion), [go] "v"(qo + kKvDRegion), [q00] "v"(tq[0]),
        [q10] "v"(tq[1]), [q01] "v"(tq[2]), [q11] "v"(tq[3]), [d00] "v"(tq[0] + kKvDRegion),
        [d10] "v"(tq[1] + kKvDRegion), [d01] "v"(tq[2] + kKvDRegion), [d11] "v"(tq[3] + kKvDRegion),
        [lp0] "v"(lp0), [lp1] "v"(lp1), [vk] "v"(uint32_t(vk)), [off] "v"(off)
      : "memory", "vcc", "scc", "m0", "s84", "s85", "s86", "s87", "s88", "s89", "s90", "s91", "s92", "s93",
        SFA_DKDV128_CLOBBER_V,
        SFA_DKDV128_CLOBBER_A);

  if (kvalid) {
    const f32x32 dk2[2] = {dka, dkb}, dv2[2] = {dva, dvb};
    const size_t krow = (size_t(base_row + vk * pstride) * p.hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 kv, vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          kv[r] = (__bf16)(dk2[db >> 1][(db & 1) * 16 + 4 * g + r] * p.scale);
          vv[r] = (__bf16)dv2[db >> 1][(db & 1) * 16 + 4 * g + r];
        }
        *reinterpret_cast<bf16x4*>(p.dk + krow + db * 32 + 8 * g + 4 * hh) = kv;
        *reinterpret_cast<bf16x4*>(p.dv + krow + db * 32 + 8 * g + 4 * hh) = vv;
      }
  }
  // the DMA of the steps past the last is still in flight: wait before the
  // work group ends and its LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// dQ at d = 128: one wave per SIMD with 64 queries (two
// blocks of 32) of one query head, so that every K / V row read from LDS
// feeds twice as many MFMAs as in bwd_dq_kernel. The work group's 4 waves
// share the key tiles: HG query heads of one key/value head times 4 / HG
// blocks of 64 queries. The tile loop is one asm stream (attn_dq128_stream.h,
// written by gen_dq128_stream.py): per 64-key tile, S^T = K Q^T and
// dP^T = V dO^T for each 32-key block, dS^T = exp2(S^T c - lse2) (dP^T - D)
// in place, rounded to bf16, and dQ^T += K^T dS^T one key block behind.
// Products, their accumulation order and the rounding of dS are those of
// bwd_dq_kernel. K and V tiles go by DMA through 3 stages (tile t + 2 while
// t runs), in the rows of 320 bytes of the d = 128 dK/dV tiles (row reads
// and transposed reads free of bank conflicts). The key tiles whose every key
// every query of the wave admits form one range per wave, tested with two
// scalar instructions; the others (the diagonal, the window's start, tiles
// past the wave's queries, and the extra tile that closes the stream) test
// each score against the lane's query.
// ---------------------------------------------------------------------------
constexpr int kDqStage = 20480;                // bytes per K (or V) stage
constexpr int kDqVRegion = 3 * kDqStage;       // V stages after the 3 K stages

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq128_kernel(BwdParams p) {
  constexpr int D = 128;
  static_assert(kDqStage == kTileBytes128, "the stream's stage offsets assume 20480-byte tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[6 * kDqStage];

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

  // work item: (batch, virtual sequence, kv head, query block, head group), heaviest first
  const int t = (blockIdx.x & 7) * p.per_xcd_q + (blockIdx.x >> 3);
  if (t >= p.total_q) return;
  const int ipu = p.nqb * p.hgroups;
  const int unit = t / ipu;
  const int rr = t - unit * ipu;
  const int qb = p.nqb - 1 - rr / p.hgroups;
  const int hg = rr % p.hgroups;
  const int kvh = unit % p.hkv;
  const int bs = unit / p.hkv;
  const int sq = bs % p.nseq;
  const int b = bs / p.nseq;
  const int h = kvh * p.G + hg * p.HG + (wave % p.HG);
  const int PS = (kWaves / p.HG) * 64;
  const int wg_q0 = qb * PS;
  const int q0 = wg_q0 + (wave / p.HG) * 64;
  const int wg_qlast = min(wg_q0 + PS, p.Lv) - 1;
  const int kt_begin = window > 0 ? max(0, wg_q0 - window + 1) / BT : 0;
  const int T = wg_qlast / BT + 1 - kt_begin;           // key tiles of the work group
  const int base_row = b * p.S + sq;

  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t dors = make_rsrc(p.dout, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lsed, p.lsed_bytes);
  const uint32_t kv_pos_bytes = uint32_t(p.hkv) * D * 2;
  const uint32_t kv_head_bytes = uint32_t(kvh) * D * 2;
  const uint32_t tstride = uint32_t(BT * pstride) * kv_pos_bytes;   // bytes between tiles

  // Q^T and dO^T (B operands: lane holds row q0 + 32 j + l32, d = 16 kk + 8 hh .. + 8),
  // and the lane's query lse2 and D
  typedef __bf16 bf16x64 __attribute__((ext_vector_type(64)));
  bf16x64 qv[2], dv[2];
  float lse2[2], dd[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vq = q0 + 32 * j + l32;
    const bool ok = vq < p.Lv;
    const uint32_t off = (uint32_t(base_row + vq * pstride) * p.hq + h) * D * 2 + 16 * hh + (ok ? 0u : kOobOffset);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 x = bload16(qrs, off + kk * 32);
      __builtin_memcpy(reinterpret_cast<char*>(&qv[j]) + kk * 16, &x, 16);
      const uint4 y = bload16(dors, off + kk * 32);
      __builtin_memcpy(reinterpret_cast<char*>(&dv[j]) + kk * 16, &y, 16);
    }
    const uint32_t li = ((uint32_t(b * p.nseq + sq) * p.hq + h) * p.Lv + vq) * 8 + (ok ? 0u : kOobOffset);
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(lrs, int(li), 0, 0);
    lse2[j] = __uint_as_float(x[0]);
    dd[j] = __uint_as_float(x[1]);
  }

  // DMA chunks of this wave: chunk w + 4 x (x < 5) of the K tile and the same
  // chunk of the V tile. Slot sl = 64 chunk + lane is 16-byte slot u = sl mod 20
  // of row sl / 20, holding data chunk u ^ row_swizzle128(row / 4); slots 16-19
  // are padding (zeros).
  uint32_t cf[5];
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const int sl = (wave + 4 * x) * 64 + lane;
    const int row = sl / 20, u = sl % 20;
    cf[x] = u >= 16 ? kOobOffset
                    : uint32_t(row * pstride) * kv_pos_bytes + kv_head_bytes + (u ^ row_swizzle128(row >> 2)) * 16;
  }
  auto tile_base = [&](int kt) { return uint32_t(base_row + kt * BT * pstride) * kv_pos_bytes; };
  // tile 0 into stage 0, zeros into the K tile of stage 2 (the first iteration
  // reads its K^T as that of a tile -1, whose dS are 0), tile 1 into stage 1
  // (tile i of the loop is key tile kt_begin + i)
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const uint32_t o0 = cf[x] < kOobOffset ? cf[x] + tile_base(kt_begin) : kOobOffset;
    dma16(krs, &lds[(wave + 4 * x) * 1024], o0);
    dma16(vrs, &lds[kDqVRegion + (wave + 4 * x) * 1024], o0);
  }
#pragma unroll
  for (int x = 0; x < 5; ++x) dma16(krs, &lds[2 * kDqStage + (wave + 4 * x) * 1024], kOobOffset);
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const uint32_t o1 = (1 < T && cf[x] < kOobOffset) ? cf[x] + tile_base(kt_begin + 1) : kOobOffset;
    dma16(krs, &lds[kDqStage + (wave + 4 * x) * 1024], o1);
    dma16(vrs, &lds[kDqVRegion + kDqStage + (wave + 4 * x) * 1024], o1);
  }
  // the loop's first DMA is tile 2
#pragma unroll
  for (int x = 0; x < 5; ++x) cf[x] = (2 < T && cf[x] < kOobOffset) ? cf[x] + tile_base(kt_begin + 2) : kOobOffset;

  // LDS read bases: rows of a 32-row block in the sigma order (chunks 2 kk + hh:
  // even kk from ke, odd from ko, plus 64 (kk / 2)); transposed reads for
  // (t, jj) from t<t><jj>, plus 64 db; stages and key blocks at immediate offsets
  const uint32_t lds0 = lds_addr(&lds[0]);
  const int ra = sigma(l32), rsw = row_swizzle128(ra >> 2);
  const uint32_t rb = lds0 + uint32_t(ra * kRowBytes128 + 16 * (hh ^ (rsw & 1)));
  const uint32_t ke = rb + 32 * (rsw >> 1), ko = rb + 32 - 32 * (rsw >> 1);
  const uint32_t ve = ke + kDqVRegion, vo = ko + kDqVRegion;
  uint32_t tr[4];
  {
    const int grp = lane >> 4, gi = lane & 15, vh = grp >> 1, e = gi >> 2;
    const int c0 = 2 * (grp & 1) + ((gi & 3) >> 1), half = gi & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = i & 1, jj = i >> 1;
      const int ro = jj ? 12 * vh + 4 + 8 * tt : 20 * vh + 8 * tt;
      tr[i] = lds0 + uint32_t((e + ro) * kRowBytes128 + 16 * (c0 ^ row_swizzle128(ro >> 2)) + 8 * half);
    }
  }
  const uint32_t lw = __builtin_amdgcn_readfirstlane(lds0 + uint32_t(wave) * 1024);
  const uint32_t Tn = __builtin_amdgcn_readfirstlane(uint32_t(T));
  // masks: the key tiles whose every key every query of the wave admits (key
  // <= q0 and q0 + 63 - key < W), as loop indices fd .. fd + fc - 1; the others
  // test each score (lane query vq0 / vq1, key offsets by register group in off)
  const int64_t W = window > 0 ? window : 0x7fffffff;
  auto cdiv = [](int64_t x) { return x >= 0 ? (x + BT - 1) / BT : -((-x) / BT); };   // ceil(x / 64)
  const int64_t fa = max<int64_t>(kt_begin, cdiv(int64_t(q0) + 64 - W));
  const int64_t fb = int64_t(q0) / BT - 1;
  const uint32_t fd = __builtin_amdgcn_readfirstlane(uint32_t(fa - kt_begin));
  const uint32_t fc = __builtin_amdgcn_readfirstlane(uint32_t(max<int64_t>(0, fb - fa + 1)));
  const uint32_t kb0 = __builtin_amdgcn_readfirstlane(uint32_t(kt_begin * BT));
  const uint32_t Wn = uint32_t(W);
  const uint32_t vq0 = uint32_t(q0 + l32), vq1 = uint32_t(q0 + 32 + l32);
  uint32_t off = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) off |= uint32_t(reg_key_offset(g, hh)) << (8 * g);

  // tile 0 and the zeros landed for every wave (tile 1 may still be in flight)
  asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");

  typedef float f32x32 __attribute__((ext_vector_type(32)));
  f32x32 d0a, d0b, d1a, d1b;
  asm volatile(
      SFA_DQ128_PROLOGUE
      SFA_DQ128_LOOP
      "s_waitcnt lgkmcnt(0)\n"
      "s_nop 7\n"
      "s_nop 7\n"
      : [d0a] "={a[0:31]}"(d0a), [d0b] "={a[32:63]}"(d0b), [d1a] "={a[64:95]}"(d1a), [d1b] "={a[96:127]}"(d1b),
        [cf0] "+v"(cf[0]), [cf1] "+v"(cf[1]), [cf2] "+v"(cf[2]), [cf3] "+v"(cf[3]), [cf4] "+v"(cf[4])
      : [q0] "{a[128:159]}"(qv[0]), [q1] "{a[160:191]}"(qv[1]), [o0] "{a[192:223]}"(dv[0]),
        [o1] "{a[224:255]}"(dv[1]), [c] "s"(p.c), [T] "s"(Tn), [tstride] "s"(tstride), [rk] "s"(krs),
        [rv] "s"(vrs), [lw] "s"(lw), [fd] "s"(fd), [fc] "s"(fc), [kb0] "s"(kb0), [W] "s"(Wn), [l0] "v"(lse2[0]),
        [l1] "v"(lse2[1]), [d0] "v"(dd[0]), [d1] "v"(dd[1]), [vq0] "v"(vq0), [vq1] "v"(vq1), [off] "v"(off), [ke] "v"(ke), [ko] "v"(ko), [ve] "v"(ve), [vo] "v"(vo),
        [t00] "v"(tr[0]), [t10] "v"(tr[1]), [t01] "v"(tr[2]), [t11] "v"(tr[3])
      : "memory", "vcc", "scc", "m0", "s84", "s85", "s86", SFA_DQ128_CLOBBER_V);

  const f32x32 dh[2][2] = {{d0a, d0b}, {d1a, d1b}};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vq = q0 + 32 * j + l32;
    if (vq >= p.Lv) continue;
    u16* orow = p.dq + (size_t(base_row + vq * pstride) * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(dh[j][db >> 1][(db & 1) * 16 + 4 * g + r] * p.scale);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hh) = ov;
      }
  }
  // the DMA of the tiles past the last is still in flight: wait before the
  // work group ends and its LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

size_t round_up(size_t x, size_t q) { return (x + q - 1) / q * q; }

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t mode) {
  // lse2 and D for every (batch, position, query head), 8 bytes each
  (void)mode;
  return round_up(size_t(batch) * n * L * hq * 8, 256);
}

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const u16*>(a.q);
  p.k = static_cast<const u16*>(a.k);
  p.v = static_cast<const u16*>(a.v);
  p.o = static_cast<const u16*>(a.o);
  p.dout = static_cast<const u16*>(a.dout);
  p.lse = a.lse;
  p.lsed = static_cast<float*>(a.ws);
  p.dq = static_cast<u16*>(a.dq);
  p.dk = static_cast<u16*>(a.dk);
  p.dv = static_cast<u16*>(a.dv);
  p.batch = int32_t(a.batch);
  const int64_t S = int64_t(a.n) * a.L;
  p.S = int32_t(S);
  const bool intra = a.mode == 0;
  p.Lv = int32_t(intra ? a.L : S);
  p.pstride = intra ? a.n : 1;
  p.nseq = intra ? a.n : 1;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.HG = 1;
  while (p.HG * 2 <= kWaves && p.G % (p.HG * 2) == 0) p.HG *= 2;
  p.hgroups = p.G / p.HG;
  p.window = (a.mode == 2 && a.window < S) ? int32_t(a.window) : 0;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  // dQ at d = 128: 64 queries per wave (bwd_dq128_kernel), else 32
  const bool dq128 = a.d == 128;
  const int PS = (kWaves / p.HG) * (dq128 ? 64 : 32);
  p.nqb = (p.Lv + PS - 1) / PS;
  p.nkb = (p.Lv + kWaves * 32 - 1) / (kWaves * 32);
  const int64_t units = int64_t(a.batch) * p.nseq * p.hkv;
  p.total_q = int32_t(units * p.nqb * p.hgroups);
  p.per_xcd_q = (p.total_q + 7) / 8;
  p.total_k = int32_t(units * p.nkb);
  p.per_xcd_k = (p.total_k + 7) / 8;
  p.q_bytes = uint32_t(a.batch * S * a.hq * a.d * 2);
  p.kv_bytes = uint32_t(a.batch * S * a.hkv * a.d * 2);
  p.lsed_bytes = uint32_t(a.batch * S * a.hq * 8);

  const dim3 pgrid(uint32_t(a.batch * a.hq * ((S + kPrepRows - 1) / kPrepRows)));
  const dim3 qgrid(uint32_t(p.per_xcd_q) * 8u), kgrid(uint32_t(p.per_xcd_k) * 8u);
  using Kernel = void (*)(BwdParams);
  static constexpr Kernel kDq64[3] = {bwd_dq_kernel<64, 0>, bwd_dq_kernel<64, 1>, bwd_dq_kernel<64, 2>};
  static constexpr Kernel kDkdv64[3] = {bwd_dkdv_kernel<64, 0>, bwd_dkdv_kernel<64, 1>, bwd_dkdv_kernel<64, 2>};
  const int kind = intra ? 0 : (p.window > 0 ? 2 : 1);
  const int di = a.d == 128;
  if (di)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, pgrid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, pgrid, dim3(256), 0, stream, p);
  static constexpr Kernel kDkdv128[3] = {bwd_dkdv128_stream_kernel<0>, bwd_dkdv128_stream_kernel<1>,
                                         bwd_dkdv128_stream_kernel<2>};
  static constexpr Kernel kDq128[3] = {bwd_dq128_kernel<0>, bwd_dq128_kernel<1>, bwd_dq128_kernel<2>};
  if (di)
    hipLaunchKernelGGL(kDkdv128[kind], kgrid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(kDkdv64[kind], kgrid, dim3(kThreads), 0, stream, p);
  if (dq128)
    hipLaunchKernelGGL(kDq128[kind], qgrid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(kDq64[kind], qgrid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfa
