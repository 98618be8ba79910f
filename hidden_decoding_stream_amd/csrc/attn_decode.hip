// Stream decode of stream-factorized attention on gfx950.
//
// What is computed: the n stream queries of the newest token T-1 in one pass
// (page "微信WeLM提出Hidden Decoding：大模型推理新范式", section 实验效果与成本分析:
// a token's n streams go through one forward pass in parallel) against the
// per-stream KV cache [batch][n][T_max][hkv][d] (aiflownews.com, section
// "Latent computation scaling and Hidden Decoding": the internal streams'
// KV cache is kept as context). Query row k sits at expanded position
// (T-1)*n + k; it sees key (t, s) at position t*n + s when the mode admits it:
//   intra        s == k (every token of its own stream)
//   cross_full   t*n + s <= (T-1)*n + k
//   cross_window the same and (T-1)*n + k - (t*n + s) < window
//
// Small-batch decode is bound by HBM bandwidth (same page and section: at
// small batch the decode is memory-bandwidth-bound and the spare compute
// absorbs the extra streams), so the design goal is to stream the cache once
// at full bandwidth:
// * A unit is one key range shared by a set of query rows: (batch, kv head)
//   with its n*G rows under the cross masks, or (batch, kv head, stream) with
//   its G rows under intra. Each unit's keys are cut into `splits` chunks; a
//   work group of 4 waves takes one chunk and each wave 32-key steps of it.
// * Keys of one stream are contiguous 32-key steps (each stream's token range
//   is padded to a multiple of 32), so a step never straddles two streams.
// * Scores use v_mfma_f32_16x16x32_bf16 as S^T = K Q^T: the K rows go from HBM
//   straight into A-operand registers (no LDS), Q^T is held in registers. The
//   two 16-key blocks of a step read keys {8g+r} and {8g+4+r} (g = lane/16)
//   so that each lane ends up holding 8 consecutive keys of one query row,
//   the B-operand layout of O^T = V^T P^T.
// * V is transposed through a per-wave LDS slab (16-byte global loads,
//   register transpose, 16-byte LDS reads), prefetched one step ahead.
// * The 4 waves of a group merge their (max, sum, O) in LDS; the group writes
//   one fp32 partial per query row and split. A second kernel merges the
//   splits in a fixed order (deterministic), rescaling by exp2(m_s - M).
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;                 // keys per wave step
constexpr int kChunkQuantum = kStep * kWaves;
constexpr int VTS = kStep + 8;            // padded row (elements) of a transposed V slab
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct DecParams {
  const u16* q;
  const u16* kc;
  const u16* vc;
  u16* o;
  float* ws_o;       // [rows][splits][d]
  float* ws_ml;      // [rows][splits][2]  (max in log2 units, sum)
  int32_t n, hq, hkv, G;
  int32_t T, Tmax, t_lo, kps;
  int32_t R;         // query rows per unit
  int32_t intra;
  int32_t window;    // 0: none
  float c;           // scale * log2(e)
  int32_t splits, chunk, keys;
};

template <int D>
struct Smem {
  union {
    u16 vt[kWaves][D * VTS];
    struct {
      float o[kWaves][16][D];
      float m[kWaves][16];
      float l[kWaves][16];
    } mrg;
  };
};

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecParams p) {
  constexpr int KC = D / 32;              // 32-wide d steps of the 16x16x32 MFMA
  constexpr int DB = D / 16;              // 16-row d blocks of O^T
  constexpr int KCH = D / 8;              // 16-byte chunks per row
  constexpr int VPL = kStep * KCH / 64;   // V chunks (keys) per lane per step
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;

  int b, kvh, s_unit;
  if (p.intra) {
    s_unit = unit % p.n;
    kvh = (unit / p.n) % p.hkv;
    b = unit / (p.n * p.hkv);
  } else {
    s_unit = 0;
    kvh = unit % p.hkv;
    b = unit / p.hkv;
  }
  // query row of this lane's B-operand column
  const int r = l16;
  const bool rvalid = r < p.R;
  const int rs = p.intra ? s_unit : (rvalid ? r / p.G : 0);     // stream of the row
  const int rh = kvh * p.G + (p.intra ? r : r % p.G);           // query head of the row
  const int pq = (p.T - 1) * p.n + rs;                           // its expanded position

  bf16x8 qf[KC];
  {
    const u16* qrow = p.q + ((size_t)(b * p.n + rs) * p.hq + (rvalid ? rh : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
      qf[kk] = rvalid ? *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + 8 * g) : bf16x8{};
  }

  const size_t stream_stride = (size_t)p.Tmax * p.hkv * D;      // elements between streams
  const u16* kbase = p.kc + (size_t)b * p.n * stream_stride + (size_t)kvh * D;
  const u16* vbase = p.vc + (size_t)b * p.n * stream_stride + (size_t)kvh * D;
  const int trow = p.hkv * D;                                   // elements between tokens

  const int j_begin = split * p.chunk;
  const int j_end = min(p.keys, j_begin + p.chunk);
  const int nsteps = j_end > j_begin ? (j_end - j_begin + kStep - 1) / kStep : 0;

  uint4 kreg[2][KC], vreg[VPL];
  auto load_step = [&](int st) {
    const int j0 = j_begin + st * kStep;
    const int sp = p.intra ? s_unit : j0 / p.kps;
    const int t0 = p.t_lo + (j0 - (j0 / p.kps) * p.kps);
    const u16* ks = kbase + (size_t)sp * stream_stride;
    const u16* vs = vbase + (size_t)sp * stream_stride;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int t = t0 + 8 * (l16 >> 2) + 4 * kb + (l16 & 3);
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        kreg[kb][kk] = t < p.T ? *reinterpret_cast<const uint4*>(ks + (size_t)t * trow + kk * 32 + 8 * g)
                               : make_uint4(0, 0, 0, 0);
    }
    const int dg = lane % KCH, kg = lane / KCH;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int t = t0 + kg * VPL + i;
      vreg[i] = t < p.T ? *reinterpret_cast<const uint4*>(vs + (size_t)t * trow + dg * 8) : make_uint4(0, 0, 0, 0);
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};

  u16* vt = sm.vt[wave];
  int st = wave;
  if (st < nsteps) load_step(st);
  for (; st < nsteps; st += kWaves) {
    const int j0 = j_begin + st * kStep;
    const int sp = p.intra ? s_unit : j0 / p.kps;
    const int t0 = p.t_lo + (j0 - (j0 / p.kps) * p.kps);

    // V: registers -> transposed LDS slab vt[d][key]
    {
      const int dg = lane % KCH, kg = lane / KCH;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(vreg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        uint32_t pk[VPL / 2];
#pragma unroll
        for (int i = 0; i < VPL / 2; ++i) {
          const uint32_t a0 = (w[(2 * i) * 4 + e / 2] >> sh) & 0xffffu;
          const uint32_t a1 = (w[(2 * i + 1) * 4 + e / 2] >> sh) & 0xffffu;
          pk[i] = a0 | (a1 << 16);
        }
        u16* dst = vt + (dg * 8 + e) * VTS + kg * VPL;
        if constexpr (VPL == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        else *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
      }
    }
    // S^T for the two 16-key blocks
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        bf16x8 a;
        __builtin_memcpy(&a, &kreg[kb][kk], 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc[kb], 0, 0, 0);
      }
    // prefetch the next step of this wave while the math runs
    if (st + kWaves < nsteps) load_step(st + kWaves);

    // mask: this lane holds keys t0 + 8g + 4kb + i of row r
    const bool edge = (t0 + kStep > p.T - 1) ||
                      (p.window > 0 && ((p.T - 1) * p.n + p.n - 1) - (t0 * p.n + sp) >= p.window);
    if (edge || !rvalid) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 8 * g + 4 * kb + i;
          const int pk = t * p.n + sp;
          bool ok = rvalid && t < p.T;
          if (!p.intra) ok = ok && pk <= pq;
          if (p.window > 0) ok = ok && pq - pk < p.window;
          if (!ok) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float cand = mx * p.c;
    const bool need = cand > m + kRescaleLog2;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - cand) : 1.f;
      if (need) m = cand;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    bf16x8 pf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], p.c, -mu));
        lsum += e;
        pf[kb * 4 + i] = (__bf16)e;
      }
    // O^T += V^T P^T: A = V^T rows d, keys 8g .. 8g+7
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (db * 16 + l16) * VTS + 8 * g);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
    }
  }

  // ---- merge the 4 waves in LDS ----
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with its V slab (the merge area aliases it)
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.mrg.o[wave][l16][db * 16 + 4 * g + i] = oacc[db][i];
  if (g == 0) {
    sm.mrg.m[wave][l16] = m;
    sm.mrg.l[wave][l16] = lsum;
  }
  __syncthreads();
  for (int idx = tid; idx < p.R * D; idx += kThreads) {
    const int row = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.mrg.m[w][row]);
    float acc = 0.f, lt = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.mrg.m[w][row] - M);
        acc += f * sm.mrg.o[w][row][d];
        lt += f * sm.mrg.l[w][row];
      }
    }
    const int rs2 = p.intra ? s_unit : row / p.G;
    const int rh2 = kvh * p.G + (p.intra ? row : row % p.G);
    const size_t orow = (size_t)(b * p.n + rs2) * p.hq + rh2;
    p.ws_o[(orow * p.splits + split) * D + d] = acc;
    if (d == 0) {
      p.ws_ml[(orow * p.splits + split) * 2 + 0] = M;
      p.ws_ml[(orow * p.splits + split) * 2 + 1] = lt;
    }
  }
}

// One wave per output row. Lanes own splits (lane, lane+64, ...) for the
// max and the normaliser, and d values (lane, lane+64) for the output; the
// split weights exp2(m_s - M) are broadcast from LDS. Every reduction runs in
// a fixed order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p, int64_t rows) {
  constexpr int kMaxSplits = 1024;
  __shared__ float wsh[4][kMaxSplits];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t orow = int64_t(blockIdx.x) * 4 + wave;
  if (orow >= rows) return;
  const float* ml = p.ws_ml + orow * p.splits * 2;
  float M = -INFINITY;
  for (int s = lane; s < p.splits; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float lt = 0.f;
  for (int s = lane; s < p.splits; s += 64) {
    const float ms = ml[2 * s];
    const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    wsh[wave][s] = f;
    lt += f * ml[2 * s + 1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float inv = 1.f / lt;
  const float* po = p.ws_o + orow * p.splits * D;
#pragma unroll
  for (int d0 = 0; d0 < D; d0 += 64) {
    float acc = 0.f;
    int s = 0;
    for (; s + 4 <= p.splits; s += 4) {
      const float a0 = po[(s + 0) * D + d0 + lane], a1 = po[(s + 1) * D + d0 + lane];
      const float a2 = po[(s + 2) * D + d0 + lane], a3 = po[(s + 3) * D + d0 + lane];
      acc += wsh[wave][s + 0] * a0;
      acc += wsh[wave][s + 1] * a1;
      acc += wsh[wave][s + 2] * a2;
      acc += wsh[wave][s + 3] * a3;
    }
    for (; s < p.splits; ++s) acc += wsh[wave][s] * po[s * D + d0 + lane];
    p.o[orow * D + d0 + lane] = __builtin_bit_cast(u16, (__bf16)(acc * inv));
  }
}

int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }

}  // namespace

DecodePlan plan_decode(int64_t batch, int32_t n, int64_t T, int32_t hq, int32_t hkv, int32_t d,
                       int32_t mode, int64_t window, int32_t num_splits) {
  DecodePlan pl{};
  const int32_t G = hq / hkv;
  const bool intra = mode == 0;
  pl.rows_per_unit = intra ? G : n * G;
  pl.units = intra ? batch * hkv * n : batch * hkv;
  // Oldest token any query may see: the earliest query (stream 0 of token T-1)
  // looks back window-1 positions.
  pl.t_lo = 0;
  if (mode == 2) {
    const int64_t oldest = (T - 1) * n - window + 1;
    if (oldest > 0) pl.t_lo = oldest / n;
  }
  pl.keys_per_stream = round_up(T - pl.t_lo, kStep);
  pl.keys = (intra ? 1 : n) * pl.keys_per_stream;
  int64_t want = num_splits;
  if (want == 0) {
    const int64_t target_groups = 1024;  // about 4 work groups per CU on 256 CUs
    want = (target_groups + pl.units - 1) / pl.units;
    want = std::min<int64_t>(want, std::max<int64_t>(1, pl.keys / 256));
  }
  want = std::max<int64_t>(1, std::min<int64_t>({want, pl.keys / kStep, int64_t(1024)}));
  pl.chunk = round_up((pl.keys + want - 1) / want, kChunkQuantum);
  pl.splits = int32_t((pl.keys + pl.chunk - 1) / pl.chunk);
  const int64_t rows = batch * n * hq;
  const size_t o_bytes = size_t(rows) * pl.splits * d * 4;
  const size_t ml_bytes = size_t(rows) * pl.splits * 2 * 4;
  pl.ws_bytes = size_t(round_up(int64_t(o_bytes), 256)) + size_t(round_up(int64_t(ml_bytes), 256));
  return pl;
}

hipError_t launch_attn_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const u16*>(a.q);
  p.kc = static_cast<const u16*>(a.kc);
  p.vc = static_cast<const u16*>(a.vc);
  p.o = static_cast<u16*>(a.o);
  const int64_t rows = a.batch * a.n * a.hq;
  const size_t o_bytes = size_t(rows) * pl.splits * a.d * 4;
  p.ws_o = static_cast<float*>(a.ws);
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.ws) + round_up(int64_t(o_bytes), 256));
  p.n = a.n;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.T = int32_t(a.T);
  p.Tmax = int32_t(a.T_max);
  p.t_lo = int32_t(pl.t_lo);
  p.kps = int32_t(pl.keys_per_stream);
  p.R = pl.rows_per_unit;
  p.intra = a.mode == 0;
  p.window = (a.mode == 2 && a.window < int64_t(a.n) * a.T) ? int32_t(a.window) : 0;
  p.c = a.scale * kLog2e;
  p.splits = pl.splits;
  p.chunk = int32_t(pl.chunk);
  p.keys = int32_t(pl.keys);
  const dim3 grid(uint32_t(pl.splits), uint32_t(pl.units));
  if (a.d == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(uint32_t((rows + 3) / 4)), dim3(256), 0, stream, p, rows);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(uint32_t((rows + 3) / 4)), dim3(256), 0, stream, p, rows);
  }
  return hipGetLastError();
}

}  // namespace sfa
