// Prefill attention of stream-factorized attention on gfx950 (bf16 MFMA).
//
// What is computed (page "微信WeLM提出Hidden Decoding：大模型推理新范式",
// section 规模化落地的工程优化, and step 2 of section 隐式序列缩放的技术细节):
// masked softmax attention over the expanded sequence of S = n*L positions,
//   O[p] = sum_q softmax_q(scale * <Q[p], K[q]>) V[q]  over the keys q the
//   mode admits:
//   intra        q <= p, same stream (q mod n == p mod n)
//   cross_full   q <= p
//   cross_window q <= p and p - q < window
//
// Design.
// * Virtual sequences. Intra attention is n independent causal problems, one
//   per stream; stream s is the strided view of positions i*n + s. Each work
//   group therefore runs a causal (optionally windowed) attention over a
//   "virtual" sequence: index i maps to position i*pstride + s, with
//   pstride = n, s = stream for intra and pstride = 1, s = 0 for the cross
//   modes. Tiles are dense in the virtual index, so intra mode spends no
//   MFMA work on the other streams' keys, and only the diagonal tile of each
//   query block needs an element mask.
// * Block skipping. A work group visits only key tiles that hold an allowed
//   pair: tiles past its last query (causal) and, for cross_window, tiles that
//   end before its first query's window are never loaded.
// * MFMA formulation. With v_mfma_f32_32x32x16_bf16 each wave computes the
//   transposed scores S^T = K Q^T (A = K rows from LDS, B = Q^T held in
//   registers), so after the MFMA a lane holds 16 keys of ONE query column.
//   Row max / row sum are then lane-local plus one exchange with lane l^32.
//   The probabilities feed O^T = V^T P^T straight from the accumulator
//   registers: K rows are read in a permuted order (sigma below) such that
//   lane half h holds keys 16h .. 16h+15 of each 32-key block. V stays
//   row-major in LDS; its A operand (V^T) is gathered with the gfx950
//   transposed LDS read ds_read_b64_tr_b16, addressed so that each lane
//   receives exactly the keys its P^T registers hold.
// * Memory. K and V tiles go from HBM to LDS by buffer->LDS DMA loads (no
//   staging registers, no LDS write instructions) through a 4-stage ring
//   worked in pairs of tiles: the first tile of a pair sends out the DMA of
//   the next pair, and one bare barrier per pair publishes it. Rows past the end of a sequence use an
//   out-of-range offset and read as zeros, with no branch. K rows are padded
//   and V pieces swizzled so that the operand reads are free of bank
//   conflicts.
// * Occupancy. A work group is 8 waves (two per SIMD), each owning 32
//   queries of one query head; one group per CU (138 KiB of LDS at d=128).
// * Online softmax in base 2 with lazy rescaling: the running reference max m
//   is raised only when a tile's max exceeds it by more than 2^8; until then
//   exp2(s - m) <= 256 and no O rescale is needed. The result is the same
//   quotient sum(p v) / sum(p) for any reference m.
// * Work order. Items (batch, stream, kv head, query block, head group) are
//   laid out so that block i runs on XCD i % 8 and each XCD owns a contiguous
//   range of items: the query heads of one kv head and neighbouring query
//   blocks run on the same XCD at the same time and share its L2. Within a
//   range the heaviest (latest) query blocks go first.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BN = 64;                    // keys per tile
constexpr float kRescaleLog2 = 8.0f;      // lazy-rescale threshold (log2 units)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

struct FwdParams {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  int32_t S;         // expanded positions per sequence
  int32_t Lv;        // keys of a virtual sequence (S cross, L intra)
  int32_t pstride;   // virtual key index -> position stride (1 cross, n intra)
  int32_t nseq;      // virtual sequences per batch element (1 cross, n intra)
  int32_t sq0;       // stream of the first virtual sequence (intra)
  // Queries. Query iq of virtual sequence sq sits in Q / O row
  // b*QS + sq*q_sq + iq*q_rs and on key index iq*qn + qoff (its diagonal).
  int32_t Lq;        // queries per virtual sequence
  int32_t QS, q_sq, q_rs;
  int32_t qn, qoff;
  int32_t hq, hkv, G, HG;
  int32_t window;    // > 0: cross_window limit in positions; 0: none
  float c;           // scale * log2(e)
  int32_t nqb;       // query blocks per virtual sequence
  int32_t hgroups;   // G / HG
  int32_t total;     // work items
  int32_t per_xcd;   // ceil(total / 8)
  uint32_t q_bytes;  // buffer sizes (<= 2^31) for out-of-range checks
  uint32_t kv_bytes;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// All V^T fragments of a tile in one asm block of ds_read_b64_tr_b16,
// which also waits for them: output i = ((db*2 + kb)*2 + j2)*2 + tr reads
// key row kb*32 + 4*(2*tr + j2) (+ the lane's row within its group) of the
// 32-wide d block db, from base ae[db] (j2 = 0) or ao[db] (j2 = 1) plus an
// immediate offset. Through the builtin, the compiler cannot tell which LDS
// a transposed read touches and waits for every buffer->LDS load in flight
// before it, which would drain the DMA of the next tiles on every tile.
template <int D> __device__ __forceinline__ void gather_vt(u32x2 (&x)[D / 4], const uint32_t (&ae)[D / 32],
                                                          const uint32_t (&ao)[D / 32]);
template <> __device__ __forceinline__ void gather_vt<128>(u32x2 (&x)[32], const uint32_t (&ae)[4],
                                                          const uint32_t (&ao)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %32 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %32 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %36 offset:1024\n\t"
      "ds_read_b64_tr_b16 %3, %36 offset:3072\n\t"
      "ds_read_b64_tr_b16 %4, %32 offset:8192\n\t"
      "ds_read_b64_tr_b16 %5, %32 offset:10240\n\t"
      "ds_read_b64_tr_b16 %6, %36 offset:9216\n\t"
      "ds_read_b64_tr_b16 %7, %36 offset:11264\n\t"
      "ds_read_b64_tr_b16 %8, %33 offset:0\n\t"
      "ds_read_b64_tr_b16 %9, %33 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %37 offset:1024\n\t"
      "ds_read_b64_tr_b16 %11, %37 offset:3072\n\t"
      "ds_read_b64_tr_b16 %12, %33 offset:8192\n\t"
      "ds_read_b64_tr_b16 %13, %33 offset:10240\n\t"
      "ds_read_b64_tr_b16 %14, %37 offset:9216\n\t"
      "ds_read_b64_tr_b16 %15, %37 offset:11264\n\t"
      "ds_read_b64_tr_b16 %16, %34 offset:0\n\t"
      "ds_read_b64_tr_b16 %17, %34 offset:2048\n\t"
      "ds_read_b64_tr_b16 %18, %38 offset:1024\n\t"
      "ds_read_b64_tr_b16 %19, %38 offset:3072\n\t"
      "ds_read_b64_tr_b16 %20, %34 offset:8192\n\t"
      "ds_read_b64_tr_b16 %21, %34 offset:10240\n\t"
      "ds_read_b64_tr_b16 %22, %38 offset:9216\n\t"
      "ds_read_b64_tr_b16 %23, %38 offset:11264\n\t"
      "ds_read_b64_tr_b16 %24, %35 offset:0\n\t"
      "ds_read_b64_tr_b16 %25, %35 offset:2048\n\t"
      "ds_read_b64_tr_b16 %26, %39 offset:1024\n\t"
      "ds_read_b64_tr_b16 %27, %39 offset:3072\n\t"
      "ds_read_b64_tr_b16 %28, %35 offset:8192\n\t"
      "ds_read_b64_tr_b16 %29, %35 offset:10240\n\t"
      "ds_read_b64_tr_b16 %30, %39 offset:9216\n\t"
      "ds_read_b64_tr_b16 %31, %39 offset:11264\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15]), "=&v"(x[16]), "=&v"(x[17]), "=&v"(x[18]), "=&v"(x[19]), "=&v"(x[20]), "=&v"(x[21]), "=&v"(x[22]), "=&v"(x[23]), "=&v"(x[24]), "=&v"(x[25]), "=&v"(x[26]), "=&v"(x[27]), "=&v"(x[28]), "=&v"(x[29]), "=&v"(x[30]), "=&v"(x[31])
      : "v"(ae[0]), "v"(ae[1]), "v"(ae[2]), "v"(ae[3]), "v"(ao[0]), "v"(ao[1]), "v"(ao[2]), "v"(ao[3])
      : "memory");
}
template <> __device__ __forceinline__ void gather_vt<64>(u32x2 (&x)[16], const uint32_t (&ae)[2],
                                                          const uint32_t (&ao)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:512\n\t"
      "ds_read_b64_tr_b16 %3, %18 offset:1536\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:5120\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:4608\n\t"
      "ds_read_b64_tr_b16 %7, %18 offset:5632\n\t"
      "ds_read_b64_tr_b16 %8, %17 offset:0\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %10, %19 offset:512\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:1536\n\t"
      "ds_read_b64_tr_b16 %12, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:5120\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4608\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:5632\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
      : "v"(ae[0]), "v"(ae[1]), "v"(ao[0]), "v"(ao[1])
      : "memory");
}

// Tile layouts in LDS (elements, bf16):
//  K: BN rows of D + 16 (two 16-byte pad slots per row). A 16-byte operand
//     read is served 8 lanes from each half wave per cycle (lanes i and i+32
//     together); with this stride those 16 reads hit 16 distinct bank groups.
//  V: BN rows of D, unpadded; the 64-byte pieces of a row (32 d values) are
//     stored XOR-swizzled by row (position db ^ (row & 3) for D=128,
//     db ^ ((row >> 1) & 1) for D=64) so that a transposed read, which takes
//     64 bytes from each of 4 consecutive rows per half wave, hits 4 distinct
//     64-byte bank quarters.
template <int D> struct Tile {
  static constexpr int KROW = D + 16;
  static constexpr int KSLOTS = KROW / 8, VSLOTS = D / 8;      // 16-byte slots per row
  static constexpr int KI = BN * KSLOTS / 64, VI = BN * VSLOTS / 64;  // 1 KiB DMA chunks per tile
  static constexpr int KELEMS = BN * KROW, VELEMS = BN * D;
  static_assert(BN * KSLOTS % 64 == 0 && BN * VSLOTS % 64 == 0, "tile must be whole KiB chunks");
};
template <int D> __device__ __forceinline__ int vswz(int row) {
  if constexpr (D == 128) return row & 3;
  else return (row >> 1) & 1;
}

// Work group: 8 waves, two per SIMD, each owning 32 queries. K and V tiles
// of 64 keys go through a 4-stage LDS ring in pairs: while tiles t and t+1
// are computed, the DMA of tiles t+2 and t+3 is in flight, and one barrier
// per pair publishes them (half the barriers of one per tile: 2.5% faster at
// 32k). Per tile a wave runs
//   S^T = K Q^T (16 MFMAs) -> mask (edge tiles) -> row max -> lazy rescale
//   -> P = exp2(S - m), row sums, bf16 -> O^T += V^T P^T (16 MFMAs),
// with the V^T fragments gathered before the softmax so they arrive while it
// runs. The two waves of a SIMD come from the same work group but drift
// apart within a tile, so one's softmax overlaps the other's MFMAs.
// MODE is the mask (0 intra, 1 causal over the expanded sequence, 2 causal
// and windowed), fixed at compile time so that the masks and the position
// arithmetic of the other modes fold away. LASTQ: the queries are the last
// stream's only (one per token) against every stream's keys, so a query's
// diagonal lies at key index iq*n + n-1 rather than iq.
template <int D, int MODE, bool LASTQ>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(FwdParams p) {
  using TL = Tile<D>;
  constexpr int KD = D / 16;              // 16-wide d steps of Q K^T
  constexpr int DB = D / 32;              // 32-row d blocks of O^T
  constexpr int NCH = TL::KI + TL::VI;    // DMA chunks per tile (K then V)
  constexpr int NCW = (NCH + kWaves - 1) / kWaves;   // chunks per wave (max)
  constexpr int ST = 4;                   // LDS stages

  __shared__ __attribute__((aligned(16))) u16 ks[ST][TL::KELEMS];
  __shared__ __attribute__((aligned(16))) u16 vs[ST][TL::VELEMS];

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  // key index of a query's own position (the last key it may see)
  auto diag = [&](int iq) { return LASTQ ? iq * p.qn + p.qoff : iq; };

  const int tid = threadIdx.x;
  // wave index as a wave-uniform (scalar) value, so that per-wave decisions
  // below are scalar branches rather than exec-mask branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item ----
  const int t = (blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (t >= p.total) return;
  const int ipu = p.nqb * p.hgroups;
  const int unit = t / ipu;
  const int rr = t - unit * ipu;
  const int qb = p.nqb - 1 - rr / p.hgroups;
  const int hg = rr % p.hgroups;
  const int kvh = unit % p.hkv;
  const int bs = unit / p.hkv;
  const int sq = p.sq0 + bs % p.nseq;
  const int b = bs / p.nseq;
  const int h = kvh * p.G + hg * p.HG + (wave % p.HG);
  const int PS = (kWaves / p.HG) * 32;
  const int wg_q0 = qb * PS;
  const int q0 = wg_q0 + (wave / p.HG) * 32;
  const int wg_qlast = min(wg_q0 + PS, p.Lq) - 1;
  const int kt_begin = window > 0 ? max(0, diag(wg_q0) - window + 1) / BN : 0;
  const int kt_end = diag(wg_qlast) / BN + 1;

  const int base_row = b * p.S + sq;       // position of virtual key index 0
  const int qbase_row = b * p.QS + sq * p.q_sq;   // Q / O row of query 0
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const uint32_t kv_pos_bytes = uint32_t(p.hkv) * D * 2;      // bytes between positions in K/V
  const uint32_t kv_head_bytes = uint32_t(kvh) * D * 2;

  // ---- Q^T fragments (B operand): lane holds Q[q0+l32][kk*16 + 8*hh .. +8] ----
  bf16x8 qf[KD];
  {
    const int vq = q0 + l32;
    const uint32_t off = ((uint32_t(qbase_row + vq * p.q_rs) * p.hq + h) * D + 8 * hh) * 2 +
                         (vq < p.Lq ? 0u : kOobOffset);
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const uint4 x = bload16(qrs, off + kk * 32);
      __builtin_memcpy(&qf[kk], &x, 16);
    }
  }

  // ---- tile staging: global -> LDS by DMA ----
  // Chunk c < KI is K chunk c (slot sl = 64 c + lane of the padded K tile:
  // row sl / KSLOTS, data chunk sl % KSLOTS, padding reads zeros); chunk
  // c >= KI is V chunk c - KI (row sl / VSLOTS, stored 16-byte unit
  // sl % VSLOTS, holding a data chunk of the swizzled 64-byte piece).
  // Wave w moves chunks w, w + 8, ... The byte offset of a chunk is a
  // tile-independent part (kept per chunk; padding slots carry the
  // out-of-range offset for good) plus a scalar tile base.
  uint32_t coff[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int c = wave + j * kWaves;
    int row = 0, ch = 0;
    bool pad = false;
    if (c < TL::KI) {
      const int sl = c * 64 + lane;
      row = sl / TL::KSLOTS;
      ch = sl % TL::KSLOTS;
      pad = ch >= D / 8;
    } else {
      const int sl = (c - TL::KI) * 64 + lane;
      row = sl / TL::VSLOTS;
      const int u = sl % TL::VSLOTS;
      ch = (((u >> 2) ^ vswz<D>(row)) << 2) | (u & 3);
    }
    coff[j] = pad ? kOobOffset : uint32_t(row * pstride) * kv_pos_bytes + kv_head_bytes + ch * 16;
  }
  auto issue_chunks = [&](int kt, int j0, int j1) {
    const int st = kt % ST;
    const uint32_t tbase = uint32_t(base_row + kt * BN * pstride) * kv_pos_bytes;
    const bool ragged = (kt + 1) * BN > p.Lv;   // last tile of a sequence: rows past the end read zeros
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int c = wave + j * kWaves;
      if (c < NCH) {
        uint32_t off = tbase + coff[j];
        if (ragged) {
          const int row = c < TL::KI ? (c * 64 + lane) / TL::KSLOTS : ((c - TL::KI) * 64 + lane) / TL::VSLOTS;
          off += kt * BN + row < p.Lv ? 0u : kOobOffset;
        }
        if (c < TL::KI) dma16(krs, &ks[st][c * 512], off);
        else dma16(vrs, &vs[st][(c - TL::KI) * 512], off);
      }
    }
  };

  // K row (within a 32-key block) this lane reads for the S^T A operand.
  const int krow0 = sigma(l32);
  // Transposed V reads: lane i of 16-lane group G gathers d = 16*(G%2) + i and
  // sources row base + i/4 at column 4*(i%4) of its 64-byte piece, for its
  // group's 4 keys. The 4-key group of registers (2*j2 + t) of lane half h
  // starts at key 16h + 4*((2t + j2) ^ h); its offset from the h = 0 case is
  // 20 rows when 2t + j2 is even and 12 rows when odd. The swizzle of the
  // piece depends only on (row & 3) = i/4 (D=128) or on bit 1 of it (D=64).
  const int grp = lane >> 4, gi = lane & 15;
  const int vh = grp >> 1;
  const int vsw = D == 128 ? (gi >> 2) : ((gi >> 3) & 1);
  const int vbase = (gi >> 2) * D + 16 * (grp & 1) + 4 * (gi & 3);
  const int vbase_even = vbase + vh * 20 * D;
  const int vbase_odd = vbase + vh * 12 * D;
  const int qhi = min(q0 + 32, p.Lq) - 1;
  const bool wave_live = q0 < p.Lq;

  float m = -INFINITY, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // ---- prologue: tiles kt_begin and kt_begin + 1 in flight, wait for the first ----
  issue_chunks(kt_begin, 0, NCW);
  if (kt_begin + 1 < kt_end) issue_chunks(kt_begin + 1, 0, NCW);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int st = kt % ST;
    const bool first = ((kt - kt_begin) & 1) == 0;   // first tile of a pair
    const int k0 = kt * BN;
    const bool live = wave_live && k0 <= diag(qhi) && !(window > 0 && diag(q0) - (k0 + BN - 1) >= window);
    // the pair's first tile sends out the next pair: its stages held the
    // previous pair, which every wave finished before the last barrier
    if (first) {
      if (kt + 2 < kt_end) issue_chunks(kt + 2, 0, NCW);
      if (kt + 3 < kt_end) issue_chunks(kt + 3, 0, NCW);
    }
    if (live) {
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16 sacc[2];
      const u16* kr0 = &ks[st][krow0 * TL::KROW + 8 * hh];
      bf16x8 ka[2][KD];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) ka[kb][kk] = *reinterpret_cast<const bf16x8*>(kr0 + kb * 32 * TL::KROW + kk * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][kk], qf[kk], sacc[kb], 0, 0, 0);
      }
      // ---- V^T fragments by transposed LDS reads, issued while the matrix
      // cores still work on S^T (the mask below is the first use of it) ----
      bf16x8 va[DB][2][2];
      {
        const uint32_t vt = lds_addr(&vs[st][0]);
        uint32_t ae[DB], ao[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = ((db ^ vsw) - db) * 32 + db * 32;
          ae[db] = vt + uint32_t(vbase_even + col) * 2;
          ao[db] = vt + uint32_t(vbase_odd + col) * 2;
        }
        u32x2 x[D / 4];
        gather_vt<D>(x, ae, ao);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) __builtin_memcpy(&va[db][kb][j2], &x[((db * 2 + kb) * 2 + j2) * 2], 16);
      }

      const bool full = (k0 + BN - 1 <= diag(q0)) && (window == 0 || diag(qhi) - k0 < window);
      if (!full) {
        const int vq = diag(q0 + l32);
        const uint32_t lim = MODE == 2 ? uint32_t(window) : 0x80000000u;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = k0 + kb * 32 + reg_key_offset(g, hh) + r;
              // 0 <= vq - key < lim, one unsigned compare (lim 2^31: causal only)
              const bool ok = uint32_t(vq - key) < lim;
              sacc[kb][4 * g + r] = ok ? sacc[kb][4 * g + r] : -INFINITY;
            }
      }

      // ---- online softmax (base 2, lazy rescale) and O^T += V^T P^T, one
      // 32-key block at a time: block 0's VALU work needs only sacc[0], so it
      // runs while the matrix cores finish block 1's scores, and block 1's
      // runs while they work on block 0's P V. A raised reference max
      // rescales O (and l) before the block's P V. ----
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float mx = sacc[kb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        const float cand = pair_max(mx) * p.c;
        const bool need = cand > m + kRescaleLog2;
        if (__any(need)) {
          const float alpha = need ? __builtin_amdgcn_exp2f(m - cand) : 1.f;
          m = need ? cand : m;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        const float mu = m == -INFINITY ? 0.f : m;
        bf16x8 pf[2];
        float ls = 0.f;
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          bf16x8 pv;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j2 * 8 + i], p.c, -mu));
            ls += e;
            pv[i] = (__bf16)e;
          }
          pf[j2] = pv;
        }
        lsum += ls;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][kb][j2], pf[j2], oacc[db], 0, 0, 0);
      }
    }

    if (!first && kt + 1 < kt_end) {
      // the end of a pair: the next pair must have landed, then one barrier
      // publishes it (a bare one: every LDS read of this pair has been
      // consumed by an MFMA above, and there is no DMA left in flight)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
    }
  }

  // ---- epilogue: O = O^T / l, bf16; optional natural-log LSE ----
  if (!wave_live) return;
  const float lt = pair_sum(lsum);
  const int vq = q0 + l32;
  if (vq >= p.Lq) return;
  const float inv = 1.f / lt;
  const size_t prow = (size_t)(qbase_row + vq * p.q_rs);
  u16* orow = p.o + (prow * p.hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 ov;
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(oacc[db][4 * g + r] * inv);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hh) = ov;
    }
  if (p.lse && hh == 0)
    p.lse[((size_t)b * p.hq + h) * p.QS + (prow - (size_t)b * p.QS)] = (m + log2f(lt)) * kLn2;
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const u16*>(a.q);
  p.k = static_cast<const u16*>(a.k);
  p.v = static_cast<const u16*>(a.v);
  p.o = static_cast<u16*>(a.o);
  p.lse = a.lse;
  const int64_t S = int64_t(a.n) * a.L;
  p.S = int32_t(S);
  const bool intra = a.mode == 0;
  p.Lv = int32_t(intra ? a.L : S);
  p.pstride = intra ? a.n : 1;
  if (!a.last_stream) {
    // every position queries: a query shares the virtual index of its key
    p.nseq = intra ? a.n : 1;
    p.sq0 = 0;
    p.Lq = p.Lv;
    p.QS = p.S;
    p.q_sq = 1;
    p.q_rs = p.pstride;
    p.qn = 1;
    p.qoff = 0;
  } else {
    // one query per token, stream n-1's, in a dense [B][L] tensor
    p.nseq = 1;
    p.sq0 = intra ? a.n - 1 : 0;
    p.Lq = int32_t(a.L);
    p.QS = int32_t(a.L);
    p.q_sq = 0;
    p.q_rs = 1;
    p.qn = intra ? 1 : a.n;
    p.qoff = intra ? 0 : a.n - 1;
  }
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.HG = 1;
  while (p.HG * 2 <= kWaves && p.G % (p.HG * 2) == 0) p.HG *= 2;
  p.hgroups = p.G / p.HG;
  // A window at least as long as the sequence is full causal attention.
  p.window = (a.mode == 2 && a.window < S) ? int32_t(a.window) : 0;
  p.c = a.scale * kLog2e;
  const int PS = (kWaves / p.HG) * 32;
  p.nqb = (p.Lq + PS - 1) / PS;
  const int64_t total = int64_t(a.batch) * p.nseq * p.hkv * p.nqb * p.hgroups;
  p.total = int32_t(total);
  p.per_xcd = int32_t((total + 7) / 8);
  p.q_bytes = uint32_t(a.batch * p.QS * a.hq * a.d * 2);
  p.kv_bytes = uint32_t(a.batch * S * a.hkv * a.d * 2);
  const dim3 grid(uint32_t(p.per_xcd) * 8u);
  using Kernel = void (*)(FwdParams);
  // [d == 128][kind]: kinds 0-2 are the masks, 3-4 cross_full / cross_window
  // with last-stream queries (last-stream intra is plain intra on stream n-1)
  static constexpr Kernel kKernels[2][5] = {
      {attn_fwd_kernel<64, 0, false>, attn_fwd_kernel<64, 1, false>, attn_fwd_kernel<64, 2, false>,
       attn_fwd_kernel<64, 1, true>, attn_fwd_kernel<64, 2, true>},
      {attn_fwd_kernel<128, 0, false>, attn_fwd_kernel<128, 1, false>, attn_fwd_kernel<128, 2, false>,
       attn_fwd_kernel<128, 1, true>, attn_fwd_kernel<128, 2, true>}};
  int kind = intra ? 0 : (p.window > 0 ? 2 : 1);
  if (a.last_stream && !intra) kind += 2;
  hipLaunchKernelGGL(kKernels[a.d == 128][kind], grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfa
