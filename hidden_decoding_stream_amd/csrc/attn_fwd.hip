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
//   staging registers, no LDS write instructions) through a 4-stage ring,
//   two tiles ahead, one barrier per tile. Rows past the end of a sequence
//   use an out-of-range offset and read as zeros, with no branch. K rows are padded
//   and V pieces swizzled so that the operand reads are free of bank
//   conflicts.
// * Two kernels. attn_fwd128_kernel (d = 128, every position querying) runs
//   one wave per SIMD with 64 queries each and the whole tile loop as one
//   scheduled instruction stream; it is described where it is defined. The
//   rest of this header describes attn_fwd_kernel, which serves d = 64 and
//   the last-stream queries: a work group is 8 waves (two per SIMD), each
//   owning 32 queries of one query head; one group per CU (138 KiB of LDS at
//   d=128). The two waves of a SIMD run their MFMA and softmax phases in
//   opposite order (ping-pong), so that the VALU-heavy softmax of one
//   overlaps the MFMAs of the other.
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

#include <type_traits>

#include "attn_fwd128_stream.h"
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
  // divisions of the work-item decode (attn_fwd128_kernel): by nqb * hgroups,
  // hgroups, hkv and nseq
  FastDiv f_ipu, f_hg, f_hkv, f_nseq;
  unsigned long long* trace;   // trace build only (SFA_PREFILL_TRACE): 8 words per work item
};

// Timeline of a launch, compiled in only for the measurement build of the
// library (SFA_PREFILL_TRACE, libsfattn_trace.so): thread 0 of each work group
// writes 8 words at trace[item * 8]: s_memrealtime (100 MHz) when the item
// starts, when its first two tiles have landed, when its tile loop ends and
// when it ends; the HW_ID and XCC_ID registers (which CU and XCD ran it); the
// block index; and the item's key tiles.
#ifdef SFA_PREFILL_TRACE
#define SFA_TRACE_AT(slot)                                           \
  do {                                                               \
    if (tid == 0 && p.trace) p.trace[size_t(t) * 8 + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define SFA_TRACE_AT(slot) \
  do {                     \
  } while (0)
#endif

typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The MFMA phase of a tile in asm blocks, each holding MFMAs and the LDS
// reads of the next block spread over the first half of them, and waiting
// for those reads only at its end (a read left in flight past its asm block
// could land in a register the compiler has meanwhile reused). Transposed
// reads (ds_read_b64_tr_b16) are asm in any case: through the builtin the
// compiler cannot tell which LDS a read touches and waits for every
// buffer->LDS load in flight first. Wait states the compiler cannot see
// inside asm are written out: s_nop 2 before MFMAs that read VALU-written
// registers, and 20 after the score MFMAs whose results the VALU reads next.
// V^T chunk layout (8 transposed reads x[0..7]): for d blocks e0, e1 of one
// 32-key block kb, x[4e + 2j2 + tr] reads key rows kb*32 + 4*(2*tr + j2) (+
// the lane's row within its group) from base ae[e] (j2 = 0) or ao[e] (j2 = 1)
// plus an immediate offset; x[2j], x[2j+1] form MFMA operand j.
template <int D> struct PpAsm;
template <> struct PpAsm<128> {
  // P V chunk: O^T of d blocks e0, e1 += V^T P^T over one 32-key block (operands t: e0 j0, e0 j1,
  // e1 j0, e1 j1; P p0, p1 = j2 0, 1), two accumulators in turn, reading the V^T chunk of the next
  // (32-key block KB, d pair) at bases a0/b0 (d block e0) and a1/b1 (e1)
  template <int KB> static __device__ __forceinline__ void pv_mid(f32x16& o0, f32x16& o1, const bf16x8 (&t)[4],
                                                                  const bf16x8& p0, const bf16x8& p1, uint32_t a0,
                                                                  uint32_t b0, uint32_t a1, uint32_t b1, u32x2 (&x)[8]) {
    if constexpr (KB == 0) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:2048\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:3072\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:2048\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:3072\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [o0] "+v"(o0), [o1] "+v"(o1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    } else {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:8192\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:10240\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:9216\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:11264\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:8192\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:10240\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:9216\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:11264\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [o0] "+v"(o0), [o1] "+v"(o1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    }
  }
  // the last P V chunk, reading K chunk 0 (kk 0, 1 of both 32-key blocks) for the scores
  static __device__ __forceinline__ void pv_last(f32x16& o0, f32x16& o1, const bf16x8 (&t)[4], const bf16x8& p0,
                                                 const bf16x8& p1, uint32_t kb, u32x4 (&y)[4]) {
    asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
      "ds_read_b128 %[y0], %[kb] offset:0\n\t"
      "ds_read_b128 %[y1], %[kb] offset:32\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
      "ds_read_b128 %[y2], %[kb] offset:9216\n\t"
      "ds_read_b128 %[y3], %[kb] offset:9248\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [o0] "+v"(o0), [o1] "+v"(o1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
      : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [kb] "v"(kb)
      : "memory");
  }
  // K chunk 0 alone (scores without a P V before them)
  static __device__ __forceinline__ void k_first(uint32_t kb, u32x4 (&y)[4]) {
    asm volatile(
      "ds_read_b128 %[y0], %[kb] offset:0\n\t"
      "ds_read_b128 %[y1], %[kb] offset:32\n\t"
      "ds_read_b128 %[y2], %[kb] offset:9216\n\t"
      "ds_read_b128 %[y3], %[kb] offset:9248\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
      : [kb] "v"(kb)
      : "memory");
  }
  // S^T = K Q^T, kk pair C (operands a: kb0 kk, kb0 kk+1, kb1 kk, kb1 kk+1), reading K chunk C+1;
  // the last pair reads the first V^T chunk of the tile (32-key block 0, d blocks 0 and 1) for the
  // P V of the next MFMA phase and ends with the wait states for the VALU reading the scores
  template <int C> static __device__ __forceinline__ void s_step(f32x16& s0, f32x16& s1, const bf16x8 (&a)[4],
                                                                  const bf16x8& q0, const bf16x8& q1, uint32_t kb,
                                                                  u32x4 (&y)[4], uint32_t a0, uint32_t b0, uint32_t a1,
                                                                  uint32_t b1, u32x2 (&x)[8]) {
    if constexpr (C == 0) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], 0\n\t"
        "ds_read_b128 %[y0], %[kb] offset:64\n\t"
        "ds_read_b128 %[y1], %[kb] offset:96\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], 0\n\t"
        "ds_read_b128 %[y2], %[kb] offset:9280\n\t"
        "ds_read_b128 %[y3], %[kb] offset:9312\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [s0] "=&v"(s0), [s1] "=&v"(s1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [kb] "v"(kb)
        : "memory");
    } else if constexpr (C == 1) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], %[s0]\n\t"
        "ds_read_b128 %[y0], %[kb] offset:128\n\t"
        "ds_read_b128 %[y1], %[kb] offset:160\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], %[s1]\n\t"
        "ds_read_b128 %[y2], %[kb] offset:9344\n\t"
        "ds_read_b128 %[y3], %[kb] offset:9376\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [s0] "+v"(s0), [s1] "+v"(s1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [kb] "v"(kb)
        : "memory");
    } else if constexpr (C == 2) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], %[s0]\n\t"
        "ds_read_b128 %[y0], %[kb] offset:192\n\t"
        "ds_read_b128 %[y1], %[kb] offset:224\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], %[s1]\n\t"
        "ds_read_b128 %[y2], %[kb] offset:9408\n\t"
        "ds_read_b128 %[y3], %[kb] offset:9440\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [s0] "+v"(s0), [s1] "+v"(s1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [kb] "v"(kb)
        : "memory");
    } else {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], %[s0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:2048\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:3072\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], %[s1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:2048\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:3072\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 7\n\t"
        "s_nop 7\n\t"
        "s_nop 3\n\t"
        : [s0] "+v"(s0), [s1] "+v"(s1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    }
  }
};

template <> struct PpAsm<64> {
  // P V chunk: O^T of d blocks e0, e1 += V^T P^T over one 32-key block (operands t: e0 j0, e0 j1,
  // e1 j0, e1 j1; P p0, p1 = j2 0, 1), two accumulators in turn, reading the V^T chunk of the next
  // (32-key block KB, d pair) at bases a0/b0 (d block e0) and a1/b1 (e1)
  template <int KB> static __device__ __forceinline__ void pv_mid(f32x16& o0, f32x16& o1, const bf16x8 (&t)[4],
                                                                  const bf16x8& p0, const bf16x8& p1, uint32_t a0,
                                                                  uint32_t b0, uint32_t a1, uint32_t b1, u32x2 (&x)[8]) {
    if constexpr (KB == 0) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:512\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:1536\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:512\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:1536\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [o0] "+v"(o0), [o1] "+v"(o1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    } else {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:4096\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:5120\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:4608\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:5632\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:4096\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:5120\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:4608\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:5632\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [o0] "+v"(o0), [o1] "+v"(o1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    }
  }
  // the last P V chunk, reading K chunk 0 (kk 0, 1 of both 32-key blocks) for the scores
  static __device__ __forceinline__ void pv_last(f32x16& o0, f32x16& o1, const bf16x8 (&t)[4], const bf16x8& p0,
                                                 const bf16x8& p1, uint32_t kb, u32x4 (&y)[4]) {
    asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n\t"
      "ds_read_b128 %[y0], %[kb] offset:0\n\t"
      "ds_read_b128 %[y1], %[kb] offset:32\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t2], %[p0], %[o1]\n\t"
      "ds_read_b128 %[y2], %[kb] offset:5120\n\t"
      "ds_read_b128 %[y3], %[kb] offset:5152\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t1], %[p1], %[o0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p1], %[o1]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [o0] "+v"(o0), [o1] "+v"(o1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
      : [t0] "v"(t[0]), [t1] "v"(t[1]), [t2] "v"(t[2]), [t3] "v"(t[3]), [p0] "v"(p0), [p1] "v"(p1), [kb] "v"(kb)
      : "memory");
  }
  // K chunk 0 alone (scores without a P V before them)
  static __device__ __forceinline__ void k_first(uint32_t kb, u32x4 (&y)[4]) {
    asm volatile(
      "ds_read_b128 %[y0], %[kb] offset:0\n\t"
      "ds_read_b128 %[y1], %[kb] offset:32\n\t"
      "ds_read_b128 %[y2], %[kb] offset:5120\n\t"
      "ds_read_b128 %[y3], %[kb] offset:5152\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
      : [kb] "v"(kb)
      : "memory");
  }
  // S^T = K Q^T, kk pair C (operands a: kb0 kk, kb0 kk+1, kb1 kk, kb1 kk+1), reading K chunk C+1;
  // the last pair reads the first V^T chunk of the tile (32-key block 0, d blocks 0 and 1) for the
  // P V of the next MFMA phase and ends with the wait states for the VALU reading the scores
  template <int C> static __device__ __forceinline__ void s_step(f32x16& s0, f32x16& s1, const bf16x8 (&a)[4],
                                                                  const bf16x8& q0, const bf16x8& q1, uint32_t kb,
                                                                  u32x4 (&y)[4], uint32_t a0, uint32_t b0, uint32_t a1,
                                                                  uint32_t b1, u32x2 (&x)[8]) {
    if constexpr (C == 0) {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], 0\n\t"
        "ds_read_b128 %[y0], %[kb] offset:64\n\t"
        "ds_read_b128 %[y1], %[kb] offset:96\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], 0\n\t"
        "ds_read_b128 %[y2], %[kb] offset:5184\n\t"
        "ds_read_b128 %[y3], %[kb] offset:5216\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        : [s0] "=&v"(s0), [s1] "=&v"(s1), [y0] "=&v"(y[0]), [y1] "=&v"(y[1]), [y2] "=&v"(y[2]), [y3] "=&v"(y[3])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [kb] "v"(kb)
        : "memory");
    } else {
      asm volatile(
        "s_nop 2\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k0], %[q0], %[s0]\n\t"
        "ds_read_b64_tr_b16 %[x0], %[a0] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x1], %[a0] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x2], %[b0] offset:512\n\t"
        "ds_read_b64_tr_b16 %[x3], %[b0] offset:1536\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k2], %[q0], %[s1]\n\t"
        "ds_read_b64_tr_b16 %[x4], %[a1] offset:0\n\t"
        "ds_read_b64_tr_b16 %[x5], %[a1] offset:1024\n\t"
        "ds_read_b64_tr_b16 %[x6], %[b1] offset:512\n\t"
        "ds_read_b64_tr_b16 %[x7], %[b1] offset:1536\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s0], %[k1], %[q1], %[s0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[s1], %[k3], %[q1], %[s1]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 7\n\t"
        "s_nop 7\n\t"
        "s_nop 3\n\t"
        : [s0] "+v"(s0), [s1] "+v"(s1), [x0] "=&v"(x[0]), [x1] "=&v"(x[1]), [x2] "=&v"(x[2]), [x3] "=&v"(x[3]),
          [x4] "=&v"(x[4]), [x5] "=&v"(x[5]), [x6] "=&v"(x[6]), [x7] "=&v"(x[7])
        : [k0] "v"(a[0]), [k1] "v"(a[1]), [k2] "v"(a[2]), [k3] "v"(a[3]), [q0] "v"(q0), [q1] "v"(q1), [a0] "v"(a0),
          [b0] "v"(b0), [a1] "v"(a1), [b1] "v"(b1)
        : "memory");
    }
  }
};


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

// Work group: 8 waves, two per SIMD (waves w and w + 4), each owning 32
// queries. Per tile a wave runs an MFMA phase (O^T += V^T P^T for the previous
// tile, 16 MFMAs, then S^T = K Q^T for this tile, 16 MFMAs) and a softmax
// phase (mask on edge tiles, one reference max for the tile's 64 keys, lazy
// rescale, P = exp2(S - m) in bf16, row sums). Waves 0-3 run MFMA then
// softmax in each tile period, waves 4-7 softmax then MFMA, so on every SIMD
// one wave keeps the matrix core busy while the other runs its softmax. K and
// V tiles of 64 keys go through a 4-stage LDS ring: the DMA of tile t+2 goes
// out at the start of period t, and one barrier per period publishes tile
// t+1.
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
#ifdef SFA_PREFILL_TRACE
  if (tid == 0 && p.trace) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    p.trace[size_t(t) * 8 + 4] = hw;
    p.trace[size_t(t) * 8 + 5] = xcc;
    p.trace[size_t(t) * 8 + 6] = blockIdx.x;
  }
#endif
  SFA_TRACE_AT(0);
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
  auto chunk_off = [&](int c, int ln) {
    int row = 0, ch = 0;
    bool pad = false;
    if (c < TL::KI) {
      const int sl = c * 64 + ln;
      row = sl / TL::KSLOTS;
      ch = sl % TL::KSLOTS;
      pad = ch >= D / 8;
    } else {
      const int sl = (c - TL::KI) * 64 + ln;
      row = sl / TL::VSLOTS;
      const int u = sl % TL::VSLOTS;
      ch = (((u >> 2) ^ vswz<D>(row)) << 2) | (u & 3);
    }
    return pad ? kOobOffset : uint32_t(row * pstride) * kv_pos_bytes + kv_head_bytes + ch * 16;
  };
  uint32_t coff[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) coff[j] = chunk_off(wave + j * kWaves, lane);
  auto issue_chunks = [&](int kt, int j0, int j1) {
    const int st = kt % ST;
    const uint32_t tbase = uint32_t(base_row + kt * BN * pstride) * kv_pos_bytes;
    const bool ragged = (kt + 1) * BN > p.Lv;   // last tile of a sequence: rows past the end read zeros
    // per chunk: its precomputed offset plus this tile's base; only the
    // ragged last tile of a sequence needs a per-row check
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

  // ---- prologue: tiles kt_begin and kt_begin + 1 in flight and landed ----
  issue_chunks(kt_begin, 0, NCW);
  if (kt_begin + 1 < kt_end) issue_chunks(kt_begin + 1, 0, NCW);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");
  SFA_TRACE_AT(1);

  // The Q fragments' loads completed at the wait above, but the compiler does
  // not read inline asm: passing them through an empty asm makes it place its
  // own wait for them here, outside the tile loop, instead of before their
  // uses inside it, where its count would also wait for the DMA in flight.
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) asm volatile("" : "+v"(qf[kk]));
  const int T = kt_end - kt_begin;
  const bool grp_b = wave >= kWaves / 2;   // waves w and w + 4 share a SIMD
  const bool full_share = wave + (NCW - 1) * kWaves < NCH;   // this wave moves NCW chunks per tile (else NCW - 1)
  auto live = [&](int kt) {
    const int k0 = kt * BN;
    return wave_live && k0 <= diag(qhi) && !(window > 0 && diag(q0) - (k0 + BN - 1) >= window);
  };
  f32x16 sacc[2];
  bf16x8 pf[4];   // P of the last softmax, [32-key block * 2 + j2]

  u32x2 xv[8];   // the first V^T chunk of the last scored tile, read ahead by its last score block
  auto vaddr = [&](int stage, uint32_t (&ae)[DB], uint32_t (&ao)[DB]) {
    const uint32_t vt = lds_addr(&vs[stage][0]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = (db ^ vsw) * 32;
      ae[db] = vt + uint32_t(vbase_even + col) * 2;
      ao[db] = vt + uint32_t(vbase_odd + col) * 2;
    }
  };
  // MFMA phase i: O^T += V^T P^T for tile i-1 in chunks of (32-key block,
  // pair of d blocks), then S^T = K Q^T for tile i in pairs of 16-wide d steps
  auto mfma_phase = [&](int i) {
    const bool do_pv = i >= 1 && live(kt_begin + i - 1);
    const bool do_s = i < T && live(kt_begin + i);
    const int sts = (kt_begin + i) % ST;
    const uint32_t kbase = lds_addr(&ks[sts][krow0 * TL::KROW + 8 * hh]);
    u32x4 y[4];
    if (do_pv) {
      uint32_t ae[DB], ao[DB];
      vaddr((kt_begin + i - 1) % ST, ae, ao);
      constexpr int NP = DB / 2;
      auto chunk = [&](auto CC) {
        constexpr int c = decltype(CC)::value;
        constexpr int kb = c / NP, pr = c % NP;
        bf16x8 t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) __builtin_memcpy(&t[j], &xv[2 * j], 16);
        if constexpr (c + 1 < 2 * NP) {
          constexpr int kbn = (c + 1) / NP, prn = (c + 1) % NP;
          PpAsm<D>::template pv_mid<kbn>(oacc[2 * pr], oacc[2 * pr + 1], t, pf[2 * kb], pf[2 * kb + 1], ae[2 * prn],
                                         ao[2 * prn], ae[2 * prn + 1], ao[2 * prn + 1], xv);
        } else {
          PpAsm<D>::pv_last(oacc[2 * pr], oacc[2 * pr + 1], t, pf[2 * kb], pf[2 * kb + 1], kbase, y);
        }
      };
      chunk(std::integral_constant<int, 0>{});
      chunk(std::integral_constant<int, 1>{});
      if constexpr (D == 128) {
        chunk(std::integral_constant<int, 2>{});
        chunk(std::integral_constant<int, 3>{});
      }
    } else if (do_s) {
      PpAsm<D>::k_first(kbase, y);
    }
    if (do_s) {
      uint32_t ae[DB], ao[DB];
      vaddr(sts, ae, ao);
      auto step = [&](auto C) {
        constexpr int c = decltype(C)::value;
        bf16x8 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) __builtin_memcpy(&a[j], &y[j], 16);
        PpAsm<D>::template s_step<c>(sacc[0], sacc[1], a, qf[2 * c], qf[2 * c + 1], kbase, y, ae[0], ao[0], ae[1],
                                     ao[1], xv);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      if constexpr (D == 128) {
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
      }
    }
  };

  // softmax phase i: mask, one reference max for the 64 keys of the tile
  // (lazy rescale), P = exp2(S - m) in bf16, row sums
  auto softmax_phase = [&](int i) {
    const int kt = kt_begin + i;
    if (!live(kt)) return;
    const int k0 = kt * BN;
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
            const bool ok = uint32_t(vq - key) < lim;
            sacc[kb][4 * g + r] = ok ? sacc[kb][4 * g + r] : -INFINITY;
          }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[0][j]);
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[1][j]);
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
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        bf16x8 pv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j2 * 8 + j], p.c, -mu));
          ls += e;
          pv[j] = (__bf16)e;
        }
        pf[kb * 2 + j2] = pv;
      }
    lsum += ls;
  };

  // Period pp: group A (waves 0-3) runs the MFMA phase of tile pp then the
  // softmax of tile pp; group B (waves 4-7) the softmax of tile pp-1 then the
  // MFMA phase of tile pp. On each SIMD one wave multiplies while the other
  // runs its softmax. The DMA of tile pp+2 goes out at the start of the
  // period into the stage tile pp-2 held, which both groups finished reading
  // in period pp-1.
  auto period_end = [&](int pp) {
    if (pp + 1 < T) {
      // tile pp+1 must have landed; the chunks of tile pp+2 may still fly
      if (pp + 2 < T) {
        if (full_share) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCW) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCW - 1) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_barrier" ::: "memory");
    }
  };
  // one loop per group (the same barriers in both): a single loop with both
  // orders would carry each group's state through the other's path
  if (!grp_b) {
#pragma nounroll
    for (int pp = 0; pp <= T; ++pp) {
      if (pp + 2 < T) issue_chunks(kt_begin + pp + 2, 0, NCW);
      mfma_phase(pp);
      if (pp < T) softmax_phase(pp);
      period_end(pp);
    }
  } else {
#pragma nounroll
    for (int pp = 0; pp <= T; ++pp) {
      if (pp + 2 < T) issue_chunks(kt_begin + pp + 2, 0, NCW);
      if (pp >= 1) softmax_phase(pp - 1);
      mfma_phase(pp);
      period_end(pp);
    }
  }
  // the last P V MFMAs' results are read by the VALU below
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  SFA_TRACE_AT(2);
#ifdef SFA_PREFILL_TRACE
  if (tid == 0 && p.trace) p.trace[size_t(t) * 8 + 7] = uint32_t(T);
#endif

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
  SFA_TRACE_AT(3);
}


// ---------------------------------------------------------------------------
// d = 128, every position querying: one wave per SIMD.
//
// A work group is 4 waves (one per SIMD), each owning 64 queries (two 32-query
// blocks QB0, QB1) of one query head, with 512 registers per wave. Per 64-key
// tile t a wave issues 64 MFMAs in one scheduled instruction stream:
//   S0(t)  = K(t) Q0^T             (16, scores of QB0)
//   O1    += V(t-1)^T P1(t-1)^T    (16, QB1's P V of the previous tile)
//   S1(t)  = K(t) Q1^T             (16)
//   O0    += V(t)^T P0(t)^T        (16)
// and in the shadow of each MFMA (32 cycles) up to 7 other instructions: the
// softmax of QB0 of tile t between S0(t) and O0 += ..., that of QB1 between
// S1(t) and the next tile's O1 += ..., the V^T reads of tile t (into the
// registers each finished O1 MFMA frees), the K reads of tile t+1, the
// barrier and the DMA of tile t+4. K operands are read once per tile for 64
// queries, half the LDS reads per query of the two-waves-per-SIMD kernel.
// The whole tile loop is one asm block (the stream, its register plan and
// the wait states between its instructions are fixed, see the block's
// layout below), unrolled over the 4 LDS stages so that every LDS offset is
// an immediate.
//
// Register plan (per wave): AGPR a0-63 O0^T, a64-127 O1^T (4 d blocks x 16),
// a128-159 / a160-191 Q0^T / Q1^T (8 k steps x 4), a192-255 V^T operands of
// one tile (4 d blocks x 2 key blocks x 2 k steps); VGPR v96-159 K operands of
// one tile (2 key blocks x 8 k steps), v160-175 / v176-191 P1 / P0 in bf16,
// v192-223 / v224-255 S1 / S0, v80-95 temporaries.
//
// Softmax. The probabilities of a tile are computed against the running
// reference max m as they stand, p = exp2(c s - m), summed per lane from the
// bf16 values the P V product uses (v_dot2 with ones). Only when a lane's sum
// over the tile exceeds 2^8, which any p > 2^8 implies, does the wave take the
// out-of-line path: it forms the tile's max, raises m where the max exceeds
// it by more than 2^8 (rescaling O and l there) and recomputes the tile. This
// is the lazy rescale of the two-waves kernel with its per-tile max taken
// only when it can matter.
//
// Masks: a tile is full (every key allowed for every query of the block),
// empty, or one of at most three special tiles per query block (the
// diagonal, and up to two tiles cut by the window's start), whose per-lane
// 32-bit mask words are formed once per work item. Full tiles cost one
// scalar compare; the rest go out of line and set masked scores to -inf.
//
// Memory: K (rows of 320 bytes, 16-byte chunks swizzled by row quad) and V
// (64-byte pieces swizzled by row) tiles go from HBM to LDS by DMA through 4
// stages of 36 KiB; every wave moves 5 K and 4 V chunks of 1 KiB per tile, so
// that the wait for tile t+1 before the barrier of tile t is one fixed count. Past the last tile the
// DMA continues with out-of-range offsets (zeros), and the loop runs one
// extra, fully masked, tile so that the last tile's QB1 P V runs in the same
// stream; rows past the end of a sequence load the next rows of the buffer
// (or zeros past its end), which the causal mask excludes.
constexpr int kW128 = 4;
constexpr int kKStage128 = 20480;         // LDS bytes per K stage (64 rows of 320)
constexpr int kVStage128 = 16384;         // per V stage
constexpr int kVRegion128 = 4 * kKStage128;   // the 4 V stages follow the 4 K stages

template <int MODE>
__global__ __launch_bounds__(64 * kW128, 1) void attn_fwd128_kernel(FwdParams p) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * (kKStage128 + kVStage128)];

  const int pstride = MODE == 0 ? p.pstride : 1;
  const int window = MODE == 2 ? p.window : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  // ---- work item: (batch, stream, kv head, query block, head group) ----
  const int t = (blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (t >= p.total) return;
#ifdef SFA_PREFILL_TRACE
  if (tid == 0 && p.trace) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    p.trace[size_t(t) * 8 + 4] = hw;
    p.trace[size_t(t) * 8 + 5] = xcc;
    p.trace[size_t(t) * 8 + 6] = blockIdx.x;
  }
#endif
  SFA_TRACE_AT(0);
  const int unit = int(fdiv(uint32_t(t), p.f_ipu));
  const int rr = t - unit * int(p.f_ipu.d);
  const int rq = int(fdiv(uint32_t(rr), p.f_hg));
  const int qb = p.nqb - 1 - rq;
  const int hg = rr - rq * p.hgroups;
  const int bs = int(fdiv(uint32_t(unit), p.f_hkv));
  const int kvh = unit - bs * p.hkv;
  const int b = int(fdiv(uint32_t(bs), p.f_nseq));
  const int sq = p.sq0 + bs - b * p.nseq;
  const int h = kvh * p.G + hg * p.HG + (wave % p.HG);
  const int PS = (kW128 / p.HG) * 64;
  const int wg_q0 = qb * PS;
  const int q0 = wg_q0 + (wave / p.HG) * 64;
  const int wg_qlast = min(wg_q0 + PS, p.Lq) - 1;
  const int kt_begin = window > 0 ? max(0, wg_q0 - window + 1) / BN : 0;
  const int kt_end = wg_qlast / BN + 1;
  const int T = kt_end - kt_begin;

  const int base_row = b * p.S + sq;
  const int qbase_row = b * p.QS + sq * p.q_sq;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const uint32_t kv_pos_bytes = uint32_t(p.hkv) * D * 2;
  const uint32_t kv_head_bytes = uint32_t(kvh) * D * 2;
  const uint32_t tstride = uint32_t(BN * pstride) * kv_pos_bytes;   // bytes between tiles

  // ---- Q^T fragments: lane holds Q[q0 + 32 j + l32][kk*16 + 8 hh .. +8] ----
  typedef __bf16 bf16x64 __attribute__((ext_vector_type(64)));
  bf16x64 qv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vq = q0 + 32 * j + l32;
    const uint32_t off = ((uint32_t(qbase_row + vq * p.q_rs) * p.hq + h) * D + 8 * hh) * 2 +
                         (vq < p.Lq ? 0u : kOobOffset);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 x = bload16(qrs, off + kk * 32);
      __builtin_memcpy(reinterpret_cast<char*>(&qv[j]) + kk * 16, &x, 16);
    }
  }
  // (the Q loads complete with the first tile, at the wait before the loop)

  // ---- DMA chunks of this wave: K chunks w + 4j (j < 5), V chunks w + 4(j - 5) ----
  // A K row is 20 slots of 16 bytes: slot u < 16 holds data chunk
  // u ^ row_swizzle128(row / 4) (the K reads below are then free of bank
  // conflicts), slots 16-19 are padding (zeros).
  uint32_t cf[9];
#pragma unroll
  for (int jx = 0; jx < 9; ++jx) {
    if (jx < 5) {
      const int sl = (wave + 4 * jx) * 64 + lane;
      const int row = sl / 20, u = sl % 20;
      cf[jx] = u >= 16 ? kOobOffset
                       : uint32_t(row * pstride) * kv_pos_bytes + kv_head_bytes +
                             (u ^ row_swizzle128(row >> 2)) * 16;
    } else {
      const int sl = (wave + 4 * (jx - 5)) * 64 + lane;
      const int row = sl / 16, u = sl % 16;
      const int ch = (((u >> 2) ^ (row & 3)) << 2) | (u & 3);
      cf[jx] = uint32_t(row * pstride) * kv_pos_bytes + kv_head_bytes + ch * 16;
    }
  }
  const uint32_t lds0 = lds_addr(&lds[0]);
  auto tile_base = [&](int kt) { return uint32_t(base_row + kt * BN * pstride) * kv_pos_bytes; };
  // tiles 0..3 of the loop into stages 0..3 (past the last tile: zeros)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t tb = tile_base(kt_begin + s);
#pragma unroll
    for (int jx = 0; jx < 9; ++jx) {
      const uint32_t dst = jx < 5 ? s * kKStage128 + (wave + 4 * jx) * 1024
                                  : kVRegion128 + s * kVStage128 + (wave + 4 * (jx - 5)) * 1024;
      const uint32_t off = (s < T && cf[jx] < kOobOffset) ? cf[jx] + tb : kOobOffset;
      dma16(jx < 5 ? krs : vrs, &lds[dst], off);
    }
  }
  // the loop's first DMA is tile 4
#pragma unroll
  for (int jx = 0; jx < 9; ++jx) cf[jx] = (4 < T && cf[jx] < kOobOffset) ? cf[jx] + tile_base(kt_begin + 4) : kOobOffset;

  // ---- masks: full range and special tiles of each query block ----
  uint32_t fd[2], fc[2], sp[2][3], mk[2][3];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qlo = q0 + 32 * j, qhi = qlo + 31;
    const int fa_hi = qlo >= BN - 1 ? (qlo - (BN - 1)) / BN : -1;
    const int fa_lo = window > 0 ? (qhi - window >= 0 ? (qhi - window) / BN + 1 : 0) : 0;
    fd[j] = uint32_t(fa_lo - kt_begin);
    fc[j] = uint32_t(max(0, fa_hi - fa_lo + 1));
    int cand[3] = {qlo / BN, -1, -1};
    if (window > 0) {
      // tiles holding keys qlo - window + 1 .. qhi - window (the window's start)
      const int a = qlo - window + 1, z = qhi - window;
      if (z >= 0) {
        const int ta = a >= 0 ? a / BN : 0, tz = z / BN;
        int n = 1;
        for (int x = ta; x <= tz && n < 3; ++x)
          if (x != cand[0]) cand[n++] = x;
      }
    }
    const int vq = qlo + l32;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      sp[j][k] = cand[k] >= kt_begin && cand[k] < kt_end ? uint32_t(cand[k] - kt_begin) : 0xffffffffu;
      // the lane's admitted keys of the tile, as offsets from its first key
      const int hi = vq - cand[k] * BN;
      const int lo = window > 0 ? hi - window + 1 : 0;
      mk[j][k] = cand[k] >= 0 ? tile_mask_word(lo, hi, hh) : 0u;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    fd[j] = __builtin_amdgcn_readfirstlane(fd[j]);
    fc[j] = __builtin_amdgcn_readfirstlane(fc[j]);
  }

  // ---- LDS read bases (the stages: immediate offsets; K stages 2, 3 from a
  // second pair of bases). K operand (kb, kk) of this lane is chunk 2 kk + hh
  // of row sigma(l32) + 32 kb: slot (2 kk + hh) ^ sw with sw the row's
  // swizzle, so even and odd kk sit at two per-lane offsets within each
  // 64-byte piece (the same for both key blocks).
  const int krow0 = sigma(l32);
  const int ksw = row_swizzle128(krow0 >> 2);
  const uint32_t krb = lds0 + uint32_t(krow0 * 320 + 16 * (hh ^ (ksw & 1)));
  const uint32_t ke0 = krb + 32 * (ksw >> 1), ko0 = krb + 32 - 32 * (ksw >> 1);
  const uint32_t ke1 = ke0 + 2 * kKStage128, ko1 = ko0 + 2 * kKStage128;
  const int grp = lane >> 4, gi = lane & 15;
  const int vh = grp >> 1, vsw = gi >> 2;
  const int vbase = (gi >> 2) * D + 16 * (grp & 1) + 4 * (gi & 3);
  uint32_t ve[4], vo[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int col = (db ^ vsw) * 32;
    ve[db] = lds0 + kVRegion128 + uint32_t(vbase + vh * 20 * D + col) * 2;
    vo[db] = lds0 + kVRegion128 + uint32_t(vbase + vh * 12 * D + col) * 2;
  }
  const uint32_t lw = __builtin_amdgcn_readfirstlane(lds0 + uint32_t(wave) * 1024);
  const uint32_t Tn = __builtin_amdgcn_readfirstlane(uint32_t(T));

  // tile 0 landed for every wave
  asm volatile("s_waitcnt vmcnt(27)\n\ts_barrier" ::: "memory");
  SFA_TRACE_AT(1);

  typedef float f32x32 __attribute__((ext_vector_type(32)));
  f32x32 o0a, o0b, o1a, o1b;
  float m0 = -1e30f, l0 = 0.f, m1 = -1e30f, l1 = 0.f;
  asm volatile(
      SFA_FWD128_PROLOGUE
      SFA_FWD128_LOOP
      "s_waitcnt lgkmcnt(0)\n"
      "s_nop 7\n"
      "s_nop 7\n"
      : [o0a] "={a[0:31]}"(o0a), [o0b] "={a[32:63]}"(o0b), [o1a] "={a[64:95]}"(o1a), [o1b] "={a[96:127]}"(o1b),
        [m0] "+v"(m0), [l0] "+v"(l0), [m1] "+v"(m1), [l1] "+v"(l1), [cf0] "+v"(cf[0]), [cf1] "+v"(cf[1]),
        [cf2] "+v"(cf[2]), [cf3] "+v"(cf[3]), [cf4] "+v"(cf[4]), [cf5] "+v"(cf[5]), [cf6] "+v"(cf[6]),
        [cf7] "+v"(cf[7]), [cf8] "+v"(cf[8])
      : [q0] "{a[128:159]}"(qv[0]), [q1] "{a[160:191]}"(qv[1]), [c] "s"(p.c), [T] "s"(Tn),
        [tstride] "s"(tstride), [rk] "s"(krs), [rv] "s"(vrs), [lw] "s"(lw), [fd0] "s"(fd[0]),
        [fc0] "s"(fc[0]), [fd1] "s"(fd[1]), [fc1] "s"(fc[1]), [sp00] "v"(sp[0][0]), [sp01] "v"(sp[0][1]),
        [sp02] "v"(sp[0][2]), [sp10] "v"(sp[1][0]), [sp11] "v"(sp[1][1]), [sp12] "v"(sp[1][2]),
        [mk00] "v"(mk[0][0]), [mk01] "v"(mk[0][1]), [mk02] "v"(mk[0][2]), [mk10] "v"(mk[1][0]),
        [mk11] "v"(mk[1][1]), [mk12] "v"(mk[1][2]), [ke0] "v"(ke0), [ko0] "v"(ko0), [ke1] "v"(ke1), [ko1] "v"(ko1), [ve0] "v"(ve[0]), [ve1] "v"(ve[1]),
        [ve2] "v"(ve[2]), [ve3] "v"(ve[3]), [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3])
      : "memory", "vcc", "scc", "m0", "s84", "s85", "s86", "s87", "s88", "s89", "s90", "s91", SFA_FWD128_CLOBBER_V,
        SFA_FWD128_CLOBBER_A);

  SFA_TRACE_AT(2);
#ifdef SFA_PREFILL_TRACE
  if (tid == 0 && p.trace) p.trace[size_t(t) * 8 + 7] = uint32_t(T);
#endif

  // ---- epilogue: O = O^T / l, bf16; optional natural-log LSE ----
  const f32x32 oh[2][2] = {{o0a, o0b}, {o1a, o1b}};
  const float mm[2] = {m0, m1}, ll[2] = {l0, l1};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float lt = pair_sum(ll[j]);
    const int vq = q0 + 32 * j + l32;
    if (vq >= p.Lq) continue;
    const float inv = 1.f / lt;
    const size_t prow = (size_t)(qbase_row + vq * p.q_rs);
    u16* orow = p.o + (prow * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(oh[j][db >> 1][(db & 1) * 16 + 4 * g + r] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hh) = ov;
      }
    if (p.lse && hh == 0)
      p.lse[((size_t)b * p.hq + h) * p.QS + (prow - (size_t)b * p.QS)] = (mm[j] + log2f(lt)) * kLn2;
  }
  // The tile loop ends with DMA of the tiles past the last still in flight
  // (they write no stage a read still needs); the wave waits for them only
  // now, behind the epilogue, and before it ends and its LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  SFA_TRACE_AT(3);
}

}  // namespace

#ifdef SFA_PREFILL_TRACE
unsigned long long* g_prefill_trace = nullptr;
#endif

hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
#ifdef SFA_PREFILL_TRACE
  p.trace = g_prefill_trace;
#else
  p.trace = nullptr;
#endif
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
  // d = 128 with every position querying: the one-wave-per-SIMD kernel
  // (4 waves of 64 queries); otherwise 8 waves of 32 queries
  const bool w128 = a.d == 128 && !a.last_stream;
  const int waves = w128 ? kW128 : kWaves;
  const int qpw = w128 ? 64 : 32;
  p.HG = 1;
  while (p.HG * 2 <= waves && p.G % (p.HG * 2) == 0) p.HG *= 2;
  p.hgroups = p.G / p.HG;
  // A window at least as long as the sequence is full causal attention.
  p.window = (a.mode == 2 && a.window < S) ? int32_t(a.window) : 0;
  p.c = a.scale * kLog2e;
  const int PS = (waves / p.HG) * qpw;
  p.nqb = (p.Lq + PS - 1) / PS;
  const int64_t total = int64_t(a.batch) * p.nseq * p.hkv * p.nqb * p.hgroups;
  p.total = int32_t(total);
  p.per_xcd = int32_t((total + 7) / 8);
  p.f_ipu = make_fastdiv(uint32_t(p.nqb * p.hgroups));
  p.f_hg = make_fastdiv(uint32_t(p.hgroups));
  p.f_hkv = make_fastdiv(uint32_t(p.hkv));
  p.f_nseq = make_fastdiv(uint32_t(p.nseq));
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
  if (w128) {
    static constexpr Kernel k128[3] = {attn_fwd128_kernel<0>, attn_fwd128_kernel<1>, attn_fwd128_kernel<2>};
    hipLaunchKernelGGL(k128[kind], grid, dim3(64 * kW128), 0, stream, p);
    return hipGetLastError();
  }
  if (a.last_stream && !intra) kind += 2;
  hipLaunchKernelGGL(kKernels[a.d == 128][kind], grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfa

#ifdef SFA_PREFILL_TRACE
// Measurement build only: prefill launches after this call record their
// timeline into `buf` (device memory of at least 64 bytes per work item;
// NULL stops recording).
extern "C" void sf_trace_prefill(void* buf) { sfa::g_prefill_trace = static_cast<unsigned long long*>(buf); }
#endif
