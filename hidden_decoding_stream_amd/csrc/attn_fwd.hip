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
//   staging registers, no LDS write instructions), double-buffered with one
//   barrier per tile. Rows past the end of a sequence use an out-of-range
//   offset and read as zeros, with no branch. LDS rows are padded so that all
//   operand reads are free of bank conflicts.
// * Occupancy. Each wave owns 32 queries; two 4-wave work groups share a CU,
//   so one wave's softmax overlaps the other's matrix-core work.
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

// Query blocks of 32 per wave and work groups per CU (occupancy hint).
#ifndef SFA_FWD_QB
#define SFA_FWD_QB 1
#endif
#ifndef SFA_FWD_OCC
#define SFA_FWD_OCC 2
#endif

constexpr int kWaves = 4;
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
  int32_t Lv;        // length of a virtual sequence (S cross, L intra)
  int32_t pstride;   // virtual index -> position stride (1 cross, n intra)
  int32_t nseq;      // virtual sequences per batch element (1 cross, n intra)
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

// Key group (4 keys) that MFMA row group m>>2 reads from the K tile. After
// S^T = K Q^T, accumulator register 4g+r of lane half h holds C row
// 8g + 4h + r, i.e. key 4*kSigmaG[2g+h] + r: keys 16h .. 16h+15 of the block.
// The 16 rows that lanes 0-15 (or 16-31) read are distinct modulo 16, which
// with a padded row of D+8 elements puts them in distinct LDS bank groups.
__device__ __forceinline__ int sigma(int m) {
  constexpr uint32_t kSigmaG = 0x63417250u;  // m>>2 = 0..7 -> 0 5 2 7 1 4 3 6 (nibbles, lowest first)
  return 4 * int((kSigmaG >> (4 * (m >> 2))) & 7u) + (m & 3);
}
// Offset (within a 32-key block) of the 4 keys held in registers 4g..4g+3 by
// lane half h: 16h + 4*(((g&1)*2 + (g>>1)) ^ h).
__device__ __forceinline__ int reg_key_offset(int g, int h) { return 16 * h + 4 * ((((g & 1) * 2 + (g >> 1))) ^ h); }
__device__ __forceinline__ float wave_max_pair(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Offset that makes a buffer load return zeros (>= every num_records used).
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes bytes [16 i, 16 i + 16) after `dst` (one contiguous KiB per wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, u16* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}

// Tile layouts in LDS (elements, bf16):
//  K: BN rows of D + 8 (one 16-byte pad slot per row): MFMA A-operand reads of
//     16 rows hit 16 distinct bank groups.
//  V: BN rows of D + 32 (four pad slots): a transposed read touches 4
//     consecutive rows x 64 bytes per half wave, and a 320-byte (D=128) or
//     192-byte (D=64) row stride puts them in 4 distinct 64-byte bank quarters.
template <int D> struct Tile {
  static constexpr int KROW = D + 8, VROW = D + 32;
  static constexpr int KSLOTS = KROW / 8, VSLOTS = VROW / 8;   // 16-byte slots per row
  static constexpr int KI = BN * KSLOTS / 64, VI = BN * VSLOTS / 64;  // 1 KiB DMA chunks per tile
  static constexpr int KELEMS = BN * KROW, VELEMS = BN * VROW;
  static_assert(BN * KSLOTS % 64 == 0 && BN * VSLOTS % 64 == 0, "tile must be whole KiB chunks");
};

template <int D, int QB>
__global__ __launch_bounds__(kThreads, SFA_FWD_OCC) void attn_fwd_kernel(FwdParams p) {
  using TL = Tile<D>;
  constexpr int KD = D / 16;              // 16-wide d steps of Q K^T
  constexpr int DB = D / 32;              // 32-row d blocks of O^T
  constexpr int PSW = 32 * QB;            // query positions per wave
  constexpr int NKW = (TL::KI + kWaves - 1) / kWaves;   // DMA chunks per wave (K)
  constexpr int NVW = (TL::VI + kWaves - 1) / kWaves;   // DMA chunks per wave (V)

  __shared__ __attribute__((aligned(16))) u16 ks[2][TL::KELEMS];
  __shared__ __attribute__((aligned(16))) u16 vs[2][TL::VELEMS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
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
  const int sq = bs % p.nseq;
  const int b = bs / p.nseq;
  const int h = kvh * p.G + hg * p.HG + (wave % p.HG);
  const int PS = (kWaves / p.HG) * PSW;
  const int wg_q0 = qb * PS;
  const int q0 = wg_q0 + (wave / p.HG) * PSW;
  const int wg_qlast = min(wg_q0 + PS, p.Lv) - 1;
  const int kt_begin = p.window > 0 ? max(0, wg_q0 - p.window + 1) / BN : 0;
  const int kt_end = wg_qlast / BN + 1;

  const int base_row = b * p.S + sq;       // position of virtual index 0
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k, p.kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v, p.kv_bytes);
  const uint32_t kv_pos_bytes = uint32_t(p.hkv) * D * 2;      // bytes between positions in K/V
  const uint32_t kv_head_bytes = uint32_t(kvh) * D * 2;

  // ---- Q^T fragments (B operand): lane holds Q[q0+qi*32+l32][kk*16 + 8*hh .. +8] ----
  bf16x8 qf[QB][KD];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int vq = q0 + qi * 32 + l32;
    const uint32_t off = vq < p.Lv ? ((uint32_t(base_row + vq * p.pstride) * p.hq + h) * D + 8 * hh) * 2 : kOobOffset;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const uint4 x = bload16(qrs, off + kk * 32);
      __builtin_memcpy(&qf[qi][kk], &x, 16);
    }
  }

  // ---- tile staging: global -> LDS by DMA ----
  // Slot s of a tile (16 bytes at element 8 s) is row s / SLOTS, chunk s % SLOTS;
  // chunks past the row's data are padding and read zeros (out-of-range offset).
  int krow[NKW], kch[NKW], vrow[NVW], vch[NVW];
#pragma unroll
  for (int j = 0; j < NKW; ++j) {
    const int s = (wave + j * kWaves) * 64 + lane;
    krow[j] = s / TL::KSLOTS;
    kch[j] = s % TL::KSLOTS;
  }
#pragma unroll
  for (int j = 0; j < NVW; ++j) {
    const int s = (wave + j * kWaves) * 64 + lane;
    vrow[j] = s / TL::VSLOTS;
    vch[j] = s % TL::VSLOTS;
  }
  auto load_tile = [&](int kt, int buf) {
    const int k0 = kt * BN;
#pragma unroll
    for (int j = 0; j < NKW; ++j) {
      const int ci = wave + j * kWaves;
      if (ci < TL::KI) {
        const int vk = k0 + krow[j];
        const bool ok = vk < p.Lv && kch[j] < D / 8;
        const uint32_t off = ok ? uint32_t(base_row + vk * p.pstride) * kv_pos_bytes + kv_head_bytes + kch[j] * 16
                                : kOobOffset;
        dma16(krs, &ks[buf][ci * 512], off);
      }
    }
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
      const int ci = wave + j * kWaves;
      if (ci < TL::VI) {
        const int vk = k0 + vrow[j];
        const bool ok = vk < p.Lv && vch[j] < D / 8;
        const uint32_t off = ok ? uint32_t(base_row + vk * p.pstride) * kv_pos_bytes + kv_head_bytes + vch[j] * 16
                                : kOobOffset;
        dma16(vrs, &vs[buf][ci * 512], off);
      }
    }
  };

  float m[QB], lsum[QB];
  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    m[qi] = -INFINITY;
    lsum[qi] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qi][db] = f32x16{};
  }

  // K row (within a 32-key block) this lane reads for the S^T A operand.
  const int krow0 = sigma(l32);
  // Transposed V reads: lane i of 16-lane group G gathers d = 16*(G%2) + i and
  // sources row base + i/4 at column 4*(i%4) for its group's 4 keys. The 4-key
  // group of registers (2*j2 + t) of lane half h starts at key
  // 16h + 4*((2t + j2) ^ h); its offset from the h = 0 case is 20 rows when
  // 2t + j2 is even and 12 rows when odd.
  const int grp = lane >> 4, gi = lane & 15;
  const int vh = grp >> 1;
  const int vbase = (gi >> 2) * TL::VROW + 16 * (grp & 1) + 4 * (gi & 3);
  const int vbase_even = vbase + vh * 20 * TL::VROW;
  const int vbase_odd = vbase + vh * 12 * TL::VROW;
  const bool wave_live = q0 < p.Lv;

  load_tile(kt_begin, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    if (kt + 1 < kt_end) load_tile(kt + 1, buf ^ 1);

    // Wave-uniform tile class: `live` if any of the wave's queries has an
    // allowed key in the tile, `full` if every (query, key) pair is allowed.
    const int k0 = kt * BN;
    const int qlo = q0, qhi = min(q0 + PSW, p.Lv) - 1;
    const bool live = wave_live && k0 <= qhi && !(p.window > 0 && qlo - (k0 + BN - 1) >= p.window);
    const bool full = (k0 + BN - 1 <= qlo) && (p.window == 0 || qhi - k0 < p.window);
    if (live) {
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16 sacc[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u16* kr = &ks[buf][(kb * 32 + krow0) * TL::KROW + 8 * hh];
        bf16x8 a[KD];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(kr + kk * 16);
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
          sacc[qi][kb] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < KD; ++kk)
            sacc[qi][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], qf[qi][kk], sacc[qi][kb], 0, 0, 0);
        }
      }
      if (!full) {
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
          const int vq = q0 + qi * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key = k0 + kb * 32 + reg_key_offset(g, hh) + r;
                const bool ok = key <= vq && (p.window == 0 || vq - key < p.window);
                sacc[qi][kb][4 * g + r] = ok ? sacc[qi][kb][4 * g + r] : -INFINITY;
              }
        }
      }

      // ---- online softmax (base 2, lazy rescale) ----
      bf16x8 pf[QB][2][2];
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[qi][kb][i]);
        mx = wave_max_pair(mx);
        const float cand = mx * p.c;
        const bool need = cand > m[qi] + kRescaleLog2;
        if (__any(need)) {
          const float alpha = need ? __builtin_amdgcn_exp2f(m[qi] - cand) : 1.f;
          m[qi] = need ? cand : m[qi];
          lsum[qi] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[qi][db] *= alpha;
        }
        const float mu = m[qi] == -INFINITY ? 0.f : m[qi];
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2) {
            bf16x8 pv;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float e = __builtin_amdgcn_exp2f(fmaf(sacc[qi][kb][j2 * 8 + i], p.c, -mu));
              ls += e;
              pv[i] = (__bf16)e;
            }
            pf[qi][kb][j2] = pv;
          }
        lsum[qi] += ls;
      }

      // ---- O^T += V^T P^T, V^T gathered by transposed LDS reads ----
      const u16* vt = &vs[buf][0];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 a[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2) {
            s16x4 x[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const int c = 2 * tt + j2;
              const int base = (c & 1) ? vbase_odd : vbase_even;
              const int off = base + (kb * 32 + 4 * c) * TL::VROW + db * 32;
              x[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vt + off));
            }
            __builtin_memcpy(&a[kb][j2], x, 16);
          }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
            for (int qi = 0; qi < QB; ++qi)
              oacc[qi][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb][j2], pf[qi][kb][j2], oacc[qi][db], 0, 0, 0);
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16; optional natural-log LSE ----
  if (!wave_live) return;
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const float lt = lsum[qi] + __shfl_xor(lsum[qi], 32);
    const int vq = q0 + qi * 32 + l32;
    if (vq >= p.Lv) continue;
    const float inv = 1.f / lt;
    const size_t prow = (size_t)(base_row + vq * p.pstride);
    u16* orow = p.o + (prow * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(oacc[qi][db][4 * g + r] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hh) = ov;
      }
    if (p.lse && hh == 0)
      p.lse[((size_t)b * p.hq + h) * p.S + (prow - (size_t)b * p.S)] = (m[qi] + log2f(lt)) * kLn2;
  }
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
  p.nseq = intra ? a.n : 1;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.HG = p.G % 4 == 0 ? 4 : (p.G % 2 == 0 ? 2 : 1);
  p.hgroups = p.G / p.HG;
  // A window at least as long as the sequence is full causal attention.
  p.window = (a.mode == 2 && a.window < S) ? int32_t(a.window) : 0;
  p.c = a.scale * kLog2e;
  constexpr int QB = SFA_FWD_QB;
  const int PS = (kWaves / p.HG) * 32 * QB;
  p.nqb = (p.Lv + PS - 1) / PS;
  const int64_t total = int64_t(a.batch) * p.nseq * p.hkv * p.nqb * p.hgroups;
  p.total = int32_t(total);
  p.per_xcd = int32_t((total + 7) / 8);
  p.q_bytes = uint32_t(a.batch * S * a.hq * a.d * 2);
  p.kv_bytes = uint32_t(a.batch * S * a.hkv * a.d * 2);
  const dim3 grid(uint32_t(p.per_xcd) * 8u);
  if (a.d == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, QB>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, QB>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfa
