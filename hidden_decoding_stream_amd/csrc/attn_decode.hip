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
//   work group of 4 waves (one per SIMD) takes one chunk and each wave every
//   4th 32-key step of it. Keys of one stream are contiguous 32-key steps
//   (each stream's token range is padded to a multiple of 32), so a step
//   never straddles two streams.
// * Memory. A step's K and V rows (32 x 2 x d x 2 bytes) go from HBM to LDS
//   by buffer->LDS DMA, each wave through its own ring of stages, so no wave
//   waits for another and no barrier is needed until the end. Every group of
//   4 lanes fetches one contiguous 64-byte piece of a row (coalesced); the
//   16-byte chunks of a row are stored XOR-swizzled by key (swk / swv) so
//   that the operand reads below hit distinct LDS banks. Rows past token T-1
//   lie outside the buffer range and read as zeros.
// * Scores use v_mfma_f32_16x16x32_bf16 as S^T = K Q^T with Q^T held in
//   registers. The two 16-key blocks of a step read keys {8g+r} and
//   {8g+4+r} (g = lane/16) so that each lane ends up holding 8 consecutive
//   keys of one query row: the B-operand layout of O^T = V^T P^T. V^T comes
//   from the row-major V stage by transposed LDS reads (ds_read_b64_tr_b16).
// * Grid: units along x, splits along y. The XCDs take consecutive groups in
//   turn, so every split index spreads over all of them. Under a paged cache
//   the units are taken longest sequence first (ranked on the device from
//   seq_lens), so that with one 128 KiB group per CU the short sequences fill
//   in behind the long ones instead of a long one running alone at the end;
//   a split wholly past its sequence's keys leaves at once.
// * The 4 waves of a group merge their (max, sum, O) in LDS. With one split
//   the group writes the normalised bf16 output; otherwise it writes one fp32
//   partial per query row and split, and a second kernel merges the splits in
//   a fixed order (deterministic), rescaling by exp2(m_s - M).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sfa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;                 // keys per wave step
constexpr int kChunkQuantum = kStep * kWaves;
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
  int32_t batch;
  float len_class;           // paged: 64 / (max_T + 1), length -> one of 64 classes
  // paged cache (T above is then the largest valid length, max_T)
  const int32_t* seq_lens;   // [batch]
  const int32_t* table;      // [batch][n][max_pages] page of each (stream, logical page)
  FastDiv page;              // tokens per page (a multiple of the step)
  int64_t max_pages, num_pages;
  size_t page_elems;         // elements per page: page * hkv * d
};

// One wave's step: 32 rows of K then 32 rows of V, d elements each.
template <int D> struct Stage {
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;           // rows per 1 KiB DMA instruction
  static constexpr int NI = kStep / RPI;        // DMA instructions per 32-row tile
  static constexpr int TILE = kStep * D;        // elements per tile
  static constexpr int NS = D == 128 ? 2 : 4;   // ring depth (32 KiB per wave either way)
};

// Chunk swizzles (16-byte chunk index XOR a function of the key's low 4 bits).
// K is read 16 bytes per lane in the MFMA A layout; LDS serves lanes i and
// i+32 together, 8 of each per cycle: keys {0-3, 8-11} (+4 or +16) at chunks
// c and c^2. swk gives those 8 keys distinct values modulo XOR 2, so the 16
// reads hit 16 distinct bank groups. V is read 8 bytes per lane by the
// transposed read, 32-byte pieces of keys {0-3, 8-11} (+4, +16) at once; swv
// puts them in 8 distinct 32-byte bank slots. Both permute the chunks of a
// 64-byte quad among themselves or move whole quads, so 4 consecutive DMA
// lanes still read one contiguous 64-byte piece of the row.
template <int D> __device__ __forceinline__ int swk(int k) {
  if constexpr (D == 128) return (k & 1) | ((k & 2) << 1) | (k & 8);
  else return ((k >> 1) & 1) | ((k >> 1) & 4);
}
template <int D> __device__ __forceinline__ int swv(int k) {
  if constexpr (D == 128) return ((k & 3) << 1) | (k & 8);
  else return (k & 2) | ((k >> 1) & 4);
}

// Key space of batch element b of a paged cache. A sequence brings its own
// length; one outside [1, max_T] gets no keys (its rows come out NaN). Its
// first visited token is rounded down to a multiple of the step so that no
// step straddles two pages (the mask drops the extra tokens).
struct SeqKeys {
  int T, t_lo, kps, keys;
};
__device__ __forceinline__ SeqKeys paged_keys(const DecParams& p, int b) {
  SeqKeys s;
  s.T = p.seq_lens[b];
  if (s.T < 1 || s.T > p.T) s.T = 0;
  s.t_lo = 0;
  if (p.window > 0) {
    const int oldest = (s.T - 1) * p.n - p.window + 1;
    if (oldest > 0) s.t_lo = (oldest / p.n) & ~(kStep - 1);
  }
  s.kps = (s.T - s.t_lo + kStep - 1) / kStep * kStep;
  s.keys = (p.intra ? 1 : p.n) * s.kps;
  return s;
}

// Paged caches: batch element of the r-th longest sequence. Lengths fall into
// 64 classes (class 0 the longest; an invalid length counts as 0), ties keep
// batch order. Units are dispatched in this order, so the longest sequences'
// groups start first and the short ones fill in behind them (longest
// processing time first): with one group per CU at a time, a long sequence
// dispatched last would otherwise run on alone at the end. One wave computes
// it, with `hist` 64 words of LDS of its own; every result is wave-uniform.
__device__ __forceinline__ int len_key(const DecParams& p, int T) {
  if (T < 1 || T > p.T) T = 0;
  return 63 - min(63, int(float(T) * p.len_class));
}
__device__ int paged_rank_to_b(const DecParams& p, int r, int lane, uint32_t* hist) {
  // one wave's LDS operations complete in order; the asm statements only keep
  // the compiler from moving the plain accesses across the atomics
  hist[lane] = 0;
  asm volatile("" ::: "memory");
  for (int c = 0; c < p.batch; c += 64)
    if (c + lane < p.batch) atomicAdd(&hist[len_key(p, p.seq_lens[c + lane])], 1u);
  asm volatile("" ::: "memory");
  const int count = int(hist[lane]);
  int incl = count;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  const int excl = incl - count;
  const int cls = __ffsll((unsigned long long)__ballot(excl <= r && r < incl)) - 1;
  int rr = r - __shfl(excl, cls);
  for (int c = 0; c < p.batch; c += 64) {
    const bool in = c + lane < p.batch && len_key(p, p.seq_lens[c + lane]) == cls;
    const unsigned long long mk = __ballot(in);
    const int cnt = __popcll(mk);
    if (rr < cnt) {
      const int below = __popcll(mk & ((1ull << lane) - 1));
      return c + __ffsll((unsigned long long)__ballot(in && below == rr)) - 1;
    }
    rr -= cnt;
  }
  return 0;   // not reached for r < batch
}

template <int D, int RB, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecParams p) {
  using SG = Stage<D>;
  constexpr int KC = D / 32;              // 32-wide d steps of the 16x16x32 MFMA
  constexpr int DB = D / 16;              // 16-row d blocks of O^T
  constexpr int NS = SG::NS;
  constexpr int NI = SG::NI;
  struct Merge {
    float o[kWaves][16][D];
    float m[kWaves][16];
    float l[kWaves][16];
  };
  // One shared array per ring stage, holding every wave's (K tile, V tile)
  // of that stage. Each unrolled step below names its stage at compile time,
  // so the compiler can tell that the DMA in flight writes another array
  // than the one being read and adds no wait for it. The merge area at the
  // end (one 16-row block at a time) aliases stage 0.
  constexpr int kStageElems = kWaves * 2 * SG::TILE;
  static_assert(sizeof(Merge) <= kStageElems * 2, "merge area must fit in stage 0");
  __shared__ __attribute__((aligned(16))) u16 st0[kStageElems];
  __shared__ __attribute__((aligned(16))) u16 st1[kStageElems];
  __shared__ __attribute__((aligned(16))) u16 st2[NS > 2 ? kStageElems : 8];
  __shared__ __attribute__((aligned(16))) u16 st3[NS > 3 ? kStageElems : 8];
  Merge& mrg = *reinterpret_cast<Merge*>(st0);
  // paged: the ranked batch element, parked here for the merge instead of
  // being held in a register through the step loop (the 64-row instance has
  // none to spare)
  __shared__ int b_park;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  // units run along x: the XCDs take consecutive work groups in turn, so the
  // groups of one split index spread over all of them. (With the split along
  // x, split 0 of every unit would land on the same few XCDs, and under mixed
  // sequence lengths split 0 carries most of the work.)
  const int unit = blockIdx.x;
  const int split = blockIdx.y;

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
  if constexpr (PAGED) {
    // longest sequences first; the histogram lives in this wave's slot of
    // stage 0, which no DMA writes before the prologue below
    b = __builtin_amdgcn_readfirstlane(
        paged_rank_to_b(p, b, lane, reinterpret_cast<uint32_t*>(st0 + wave * 2 * SG::TILE)));
    if (tid == 0) b_park = b;
  }
  // Cache length of this batch element and its key index space
  int T = p.T, t_lo = p.t_lo, kps = p.kps, keys = p.keys;
  if constexpr (PAGED) {
    const SeqKeys sk = paged_keys(p, b);
    T = sk.T;
    t_lo = sk.t_lo;
    kps = sk.kps;
    keys = sk.keys;
    // a split wholly past a shorter sequence's keys has nothing to add: it
    // leaves at once and the combine does not read its slot (split 0 always
    // runs, so an invalid length still yields its NaN rows)
    if (split > 0 && split * p.chunk >= keys) return;
  }
  // query rows of this lane's B-operand columns, one per 16-row block
  bool rvalid[RB];
  int rs[RB], rh[RB], pq[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + l16;
    rvalid[rb] = r < p.R;
    rs[rb] = p.intra ? s_unit : (rvalid[rb] ? r / p.G : 0);       // stream of the row
    rh[rb] = kvh * p.G + (p.intra ? r : r % p.G);                 // query head of the row
    pq[rb] = (T - 1) * p.n + rs[rb];                              // its expanded position
  }

  const uint32_t trow_b = uint32_t(p.hkv) * D * 2;              // bytes between tokens
  const size_t stream_stride = (size_t)p.Tmax * p.hkv * D;      // elements between streams (contiguous cache)
  const u16* kbase;
  const u16* vbase;
  const int32_t* table_b = p.table;   // paged: this sequence's block table rows
  if constexpr (PAGED) {
    kbase = p.kc + (size_t)kvh * D;
    vbase = p.vc + (size_t)kvh * D;
    table_b = p.table + (size_t)b * p.n * p.max_pages;
  } else {
    kbase = p.kc + (size_t)b * p.n * stream_stride + (size_t)kvh * D;
    vbase = p.vc + (size_t)b * p.n * stream_stride + (size_t)kvh * D;
  }

  const int j_begin = split * p.chunk;
  const int j_end = min(keys, j_begin + p.chunk);
  const int nsteps = j_end > j_begin ? (j_end - j_begin + kStep - 1) / kStep : 0;
  const int nu = nsteps > wave ? (nsteps - wave + kWaves - 1) / kWaves : 0;   // steps of this wave

  // Per-lane DMA offsets within a step (tile row r, stored chunk lane % CH,
  // fetched chunk XOR the row's swizzle).
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = i * SG::RPI + lane / SG::CH;
    const int c = lane % SG::CH;
    koff[i] = uint32_t(row) * trow_b + uint32_t(c ^ swk<D>(row)) * 16;
    voff[i] = uint32_t(row) * trow_b + uint32_t(c ^ swv<D>(row)) * 16;
  }
  // this wave's slot of ring stage S (compile-time)
  auto stage = [&](auto S) -> u16* {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return st0 + wave * 2 * SG::TILE;
    else if constexpr (st == 1) return st1 + wave * 2 * SG::TILE;
    else if constexpr (st == 2) return st2 + wave * 2 * SG::TILE;
    else return st3 + wave * 2 * SG::TILE;
  };

  auto step_pos = [&](int u, int& sp, int& t0) {
    const int j0 = j_begin + (wave + u * kWaves) * kStep;
    const int ss = j0 / kps;
    sp = p.intra ? s_unit : ss;
    t0 = t_lo + (j0 - ss * kps);
  };
  auto issue = [&](int u, auto S) {
    int sp, t0;
    step_pos(u, sp, t0);
    const u16* kb;
    const u16* vb;
    uint32_t range, sbase;
    if constexpr (PAGED) {
      // the step lies in one page: look it up; rows past token T-1 (and a
      // page index outside the pool) fall outside the range and read zeros
      const uint32_t lp = fdiv(uint32_t(t0), p.page);
      const int tp0 = int(lp * p.page.d);
      const int pg = table_b[(size_t)sp * p.max_pages + lp];
      const bool pg_ok = pg >= 0 && int64_t(pg) < p.num_pages;
      const size_t pbase = size_t(pg_ok ? pg : 0) * p.page_elems;
      kb = kbase + pbase;
      vb = vbase + pbase;
      range = pg_ok ? uint32_t(min(int(p.page.d), T - tp0)) * trow_b - uint32_t(kvh) * D * 2 : 0u;
      sbase = uint32_t(t0 - tp0) * trow_b;
    } else {
      // bytes from a stream's (token 0, kv head) to the end of token T-1's
      // rows: every row t < T lies inside, every row t >= T outside
      kb = kbase + (size_t)sp * stream_stride;
      vb = vbase + (size_t)sp * stream_stride;
      range = uint32_t(T) * trow_b - uint32_t(kvh) * D * 2;
      sbase = uint32_t(t0) * trow_b;
    }
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb, range);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vb, range);
    u16* kt = stage(S);
    u16* vt = kt + SG::TILE;
    // the step base goes into the per-lane offset: only that offset is
    // range-checked, which is what turns rows t >= T into zeros
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_nt(krs, kt + i * 512, koff[i] + sbase);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_nt(vrs, vt + i * 512, voff[i] + sbase);
  };

  float m[RB], lsum[RB];
  f32x4 oacc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{};
  }

  // Q is loaded before any DMA goes out, so the wait for it that the compiler
  // places before the first step leaves every stage in flight.
  bf16x8 qf[RB][KC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const u16* qrow = p.q + ((size_t)(b * p.n + rs[rb]) * p.hq + (rvalid[rb] ? rh[rb] : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
      qf[rb][kk] = rvalid[rb] ? *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + 8 * g) : bf16x8{};
  }
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if (nu > 0) issue(0, S0{});
  if (nu > 1) issue(1, S1{});
  if constexpr (NS > 2) {
    if (nu > 2) issue(2, S2{});
    if (nu > 3) issue(3, S3{});
  }

  auto step = [&](int u, auto S) {
    // wait for step u: the stages issued after it may stay in flight
    const int after = min(NS - 1, nu - 1 - u);
    if constexpr (NS == 2) {
      if (after >= 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NI) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (after >= 3) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(6 * NI) : "memory");
      else if (after == 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * NI) : "memory");
      else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NI) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    int sp, t0;
    step_pos(u, sp, t0);
    const u16* kt = stage(S);
    const u16* vt = kt + SG::TILE;

    // K (A operand) and V^T fragments of the whole step, shared by the row blocks
    bf16x8 ka[2][KC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 8 * (l16 >> 2) + 4 * kb + (l16 & 3);
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        ka[kb][kk] = *reinterpret_cast<const bf16x8*>(kt + key * D + ((4 * kk + g) ^ swk<D>(key)) * 8);
    }
    // V^T: per d block two transposed reads (keys 8g..8g+3, 8g+4..8g+7),
    // issued in two asm blocks of eight; whole 8-byte results are copied into
    // the operand (element-wise bf16 inserts were mis-compiled into a splat).
    bf16x8 va[DB];
#pragma unroll
    for (int half = 0; half < DB / 4; ++half) {
      uint32_t addr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int db = half * 4 + j / 2, h = j & 1;
        const int key = 8 * g + 4 * h + (l16 >> 2);
        const int chunk = 2 * db + ((l16 & 3) >> 1);
        addr[j] = lds_addr(vt + key * D + (chunk ^ swv<D>(key)) * 8 + 4 * (l16 & 1));
      }
      u32x2 x[8];
      tr_read8(x, addr);
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_memcpy(&va[half * 4 + j], &x[2 * j], 16);
    }
    // the stage may be refilled once every read of it has returned
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (u + NS < nu) issue(u + NS, S);

    f32x4 sacc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[rb][kb] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          sacc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][kk], qf[rb][kk], sacc[rb][kb], 0, 0, 0);
      }

    // mask: this lane holds keys t0 + 8g + 4kb + i of row rb*16 + l16
    const bool edge = (t0 + kStep > T - 1) ||
                      (p.window > 0 && ((T - 1) * p.n + p.n - 1) - (t0 * p.n + sp) >= p.window);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (edge || !rvalid[rb]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + 8 * g + 4 * kb + i;
            const int pk = t * p.n + sp;
            bool ok = rvalid[rb] && t < T;
            if (!p.intra) ok = ok && pk <= pq[rb];
            if (p.window > 0) ok = ok && pq[rb] - pk < p.window;
            if (!ok) sacc[rb][kb][i] = -INFINITY;
          }
      }
      float mx = fmaxf(fmaxf(fmaxf(sacc[rb][0][0], sacc[rb][0][1]), fmaxf(sacc[rb][0][2], sacc[rb][0][3])),
                       fmaxf(fmaxf(sacc[rb][1][0], sacc[rb][1][1]), fmaxf(sacc[rb][1][2], sacc[rb][1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float cand = mx * p.c;
      const bool need = cand > m[rb] + kRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m[rb] - cand) : 1.f;
        if (need) m[rb] = cand;
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
      }
      const float mu = m[rb] == -INFINITY ? 0.f : m[rb];
      bf16x8 pf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[rb][kb][i], p.c, -mu));
          lsum[rb] += e;
          pf[kb * 4 + i] = (__bf16)e;
        }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pf, oacc[rb][db], 0, 0, 0);
    }
  };
  for (int u0 = 0; u0 < nu; u0 += NS) {
    step(u0, S0{});
    if (u0 + 1 < nu) step(u0 + 1, S1{});
    if constexpr (NS > 2) {
      if (u0 + 2 < nu) step(u0 + 2, S2{});
      if (u0 + 3 < nu) step(u0 + 3, S3{});
    }
  }

  // ---- merge the 4 waves in LDS, one 16-row block at a time ----
  int b_out = b;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += __shfl_xor(lsum[rb], 16);
    lsum[rb] += __shfl_xor(lsum[rb], 32);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // every wave is done with its ring (the merge area aliases stage 0), or
    // with the previous block's merge
    __syncthreads();
    if constexpr (PAGED) {
      if (rb == 0) b_out = b_park;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) mrg.o[wave][l16][db * 16 + 4 * g + i] = oacc[rb][db][i];
    if (g == 0) {
      mrg.m[wave][l16] = m[rb];
      mrg.l[wave][l16] = lsum[rb];
    }
    __syncthreads();
    // 16 threads per row, each with EPT consecutive d values: the row's max
    // and the 4 waves' factors once per thread, every LDS read of the row in
    // one round trip, vector stores
    constexpr int EPT = D / 16;
    const int nrows = min(16, p.R - rb * 16);
    const int row = tid >> 4, d0 = (tid & 15) * EPT;
    if (row < nrows) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg.m[w][row]);
      float acc[EPT], lt = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = __builtin_amdgcn_exp2f(mrg.m[w][row] - M);
#pragma unroll
          for (int e = 0; e < EPT; ++e) acc[e] += f * mrg.o[w][row][d0 + e];
          lt += f * mrg.l[w][row];
        }
      }
      const int r = rb * 16 + row;
      const int rs2 = p.intra ? s_unit : r / p.G;
      const int rh2 = kvh * p.G + (p.intra ? r : r % p.G);
      const size_t orow = (size_t)(b_out * p.n + rs2) * p.hq + rh2;
      if (p.splits == 1) {
        // every row of a valid sequence admits at least its own key, so lt > 0
        // (an invalid paged length leaves lt = 0: NaN)
        typedef __bf16 bf16xE __attribute__((ext_vector_type(EPT)));
        bf16xE ov;
#pragma unroll
        for (int e = 0; e < EPT; ++e) ov[e] = (__bf16)(acc[e] / lt);
        *reinterpret_cast<bf16xE*>(p.o + orow * D + d0) = ov;
      } else {
        float* wo = p.ws_o + (orow * p.splits + split) * D + d0;
#pragma unroll
        for (int e = 0; e < EPT; e += 4) *reinterpret_cast<f32x4*>(wo + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
        if (d0 == 0) {
          p.ws_ml[(orow * p.splits + split) * 2 + 0] = M;
          p.ws_ml[(orow * p.splits + split) * 2 + 1] = lt;
        }
      }
    }
  }
}

// One wave per output row. For the output, lane l owns 4 consecutive d
// values (d4 = l % (D/4)) of the splits s = cls, cls + C, ... with
// cls = l / (D/4) and C = 64 / (D/4) classes; the classes are summed by lane
// exchanges at the end. Every reduction runs in a fixed order, so the result
// is deterministic.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p, int64_t rows) {
  constexpr int LPR = D / 4;              // lanes covering one split's d values
  constexpr int C = 64 / LPR;             // split classes per wave
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t orow = int64_t(blockIdx.x) * 4 + wave;
  if (orow >= rows) return;
  // splits holding a partial: all of them, or under a paged cache those that
  // reach into this row's sequence (the others left without writing)
  int ns = p.splits;
  if (p.seq_lens != nullptr) {
    const int keys = paged_keys(p, int(orow / (int64_t(p.n) * p.hq))).keys;
    ns = max(1, min(p.splits, (keys + p.chunk - 1) / p.chunk));
  }
  const float* ml = p.ws_ml + orow * p.splits * 2;
  const int d4 = lane % LPR, cls = lane / LPR;
  const float* po = p.ws_o + orow * p.splits * D + 4 * d4;
  float M = -INFINITY, lt = 0.f;
  f32x4 acc = f32x4{};
  constexpr int PF = 16;                  // splits per lane loaded up front
  if (ns <= 64 && ns <= PF * C) {
    // every load first, so that the row costs one trip to memory: split
    // `lane`'s (m, l), and the m and partial O of this lane's splits. Same
    // reductions in the same order as the loops below.
    const float mv = lane < ns ? ml[2 * lane] : -INFINITY;
    const float lv = lane < ns ? ml[2 * lane + 1] : 0.f;
    float msl[PF];
    f32x4 xs[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int s = cls + i * C;
      msl[i] = s < ns ? ml[2 * s] : -INFINITY;
      xs[i] = s < ns ? *reinterpret_cast<const f32x4*>(po + (size_t)s * D) : f32x4{};
    }
    M = mv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    lt = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M) * lv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const float f = msl[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(msl[i] - M);
      acc += f * xs[i];
    }
  } else {
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    for (int s = lane; s < ns; s += 64) {
      const float ms = ml[2 * s];
      lt += ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M) * ml[2 * s + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
#pragma unroll 8
    for (int s = cls; s < ns; s += C) {
      const float ms = ml[2 * s];
      const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      const f32x4 x = *reinterpret_cast<const f32x4*>(po + (size_t)s * D);
      acc += f * x;
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
  if (cls == 0) {
    const float inv = 1.f / lt;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[i] * inv);
    *reinterpret_cast<bf16x4*>(p.o + orow * D + 4 * d4) = ov;
  }
}

int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }

}  // namespace

DecodePlan plan_decode(int64_t batch, int32_t n, int64_t T, int32_t hq, int32_t hkv, int32_t d,
                       int32_t mode, int64_t window, int32_t num_splits, bool paged) {
  DecodePlan pl{};
  const int32_t G = hq / hkv;
  const bool intra = mode == 0;
  pl.rows_per_unit = intra ? G : n * G;
  pl.units = intra ? batch * hkv * n : batch * hkv;
  pl.t_lo = 0;
  if (!paged) {
    // Oldest token any query may see: the earliest query (stream 0 of token
    // T-1) looks back window-1 positions.
    if (mode == 2) {
      const int64_t oldest = (T - 1) * n - window + 1;
      if (oldest > 0) pl.t_lo = oldest / n;
    }
    pl.keys_per_stream = round_up(T - pl.t_lo, kStep);
  } else {
    // T is the largest length; each sequence finds its own first token on the
    // device (oldest / n rounded down to a step). Its span T_b - t_lo is below
    // 34 + (window-1)/n tokens: oldest / n > T_b - 2 - (window-1)/n and the
    // rounding takes off at most 31 more.
    int64_t span = T;
    if (mode == 2) span = std::min<int64_t>(T, 34 + (window - 1) / n);
    pl.keys_per_stream = round_up(span, kStep);
  }
  pl.keys = (intra ? 1 : n) * pl.keys_per_stream;
  int64_t want = num_splits;
  if (want == 0) {
    // A group holds 128 KiB of LDS, so one runs per CU: at most one group per
    // CU (256 groups; a second, partial round of groups would add each one's
    // fixed cost), with chunks of at least one step per wave. A unit with few
    // keys (a window, a short cache) at small batch then still spreads over
    // every CU instead of leaving most of them idle.
    const int64_t target_groups = 256;
    want = std::max<int64_t>(1, target_groups / pl.units);
    want = std::min<int64_t>(want, std::max<int64_t>(1, pl.keys / kChunkQuantum));
  }
  want = std::max<int64_t>(1, std::min<int64_t>({want, pl.keys / kStep, int64_t(1024)}));
  pl.chunk = round_up((pl.keys + want - 1) / want, kChunkQuantum);
  pl.splits = int32_t((pl.keys + pl.chunk - 1) / pl.chunk);
  const int64_t rows = batch * n * hq;
  const size_t o_bytes = size_t(rows) * pl.splits * d * 4;
  const size_t ml_bytes = size_t(rows) * pl.splits * 2 * 4;
  // one split: the split kernel writes the output itself and needs no workspace
  pl.ws_bytes = pl.splits == 1 ? 0 : size_t(round_up(int64_t(o_bytes), 256)) + size_t(round_up(int64_t(ml_bytes), 256));
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
  p.batch = int32_t(a.batch);
  p.len_class = float(64.0 / (double(a.T) + 1.0));
  const bool paged = a.seq_lens != nullptr;
  p.seq_lens = a.seq_lens;
  p.table = a.table;
  p.page = make_fastdiv(uint32_t(paged ? a.page : 1));
  p.max_pages = a.max_pages;
  p.num_pages = a.num_pages;
  p.page_elems = size_t(a.page) * a.hkv * a.d;
  const dim3 grid(uint32_t(pl.units), uint32_t(pl.splits));
  const dim3 cgrid(uint32_t((rows + 3) / 4));
  using Kernel = void (*)(DecParams);
  // [d == 128][row blocks 1, 2, 4][paged]
  static constexpr Kernel kSplit[2][3][2] = {
      {{decode_split_kernel<64, 1, false>, decode_split_kernel<64, 1, true>},
       {decode_split_kernel<64, 2, false>, decode_split_kernel<64, 2, true>},
       {decode_split_kernel<64, 4, false>, decode_split_kernel<64, 4, true>}},
      {{decode_split_kernel<128, 1, false>, decode_split_kernel<128, 1, true>},
       {decode_split_kernel<128, 2, false>, decode_split_kernel<128, 2, true>},
       {decode_split_kernel<128, 4, false>, decode_split_kernel<128, 4, true>}}};
  const int rbi = p.R <= 16 ? 0 : (p.R <= 32 ? 1 : 2);
  hipLaunchKernelGGL(kSplit[a.d == 128][rbi][paged], grid, dim3(kThreads), 0, stream, p);
  if (pl.splits > 1) {
    if (a.d == 128)
      hipLaunchKernelGGL(decode_combine_kernel<128>, cgrid, dim3(256), 0, stream, p, rows);
    else
      hipLaunchKernelGGL(decode_combine_kernel<64>, cgrid, dim3(256), 0, stream, p, rows);
  }
  return hipGetLastError();
}

}  // namespace sfa
