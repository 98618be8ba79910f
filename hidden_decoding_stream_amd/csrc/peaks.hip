// Attainable-peak microbenchmarks for MI355X (gfx950), used to state the
// roofline of the attention kernels against what this chip actually reaches
// next to its published figures:
//   sfp_read   streams a device buffer once (16-byte loads, several in flight
//              per lane) and folds it into one word per work group; the
//              bandwidth a read-only kernel such as decode can reach.
//   sfp_copy   copies a buffer (read + write), the pattern of the interleave.
//   sfp_read_slices, sfp_read_slices_lds
//              read what one decode call reads, in its pattern: for each kv
//              head (work group x) and key range (work group y), the head's
//              256-byte slice of every K and V row (rows of heads * 256 bytes),
//              by 16-byte loads into registers, or by buffer->LDS DMA through
//              a ring of stages per wave, the decode kernel's way; both with
//              the nontemporal cache policy, as the decode kernel reads.
//   sfp_decode_chain
//              the batch-1 decode call's structure with no arithmetic: the
//              pattern read by DMA ring as above, each work group then writing
//              a partial of the decode's size (16 rows x (128 + 2) floats),
//              and the partials merged per output row with the decode
//              combine's loads, either by a second kernel (the library's
//              split + combine) or inside the same launch by the last work
//              group of each kv head to finish (a device-scope release fence
//              and an atomic ticket per kv head, then an acquire fence). The
//              floor each structure puts under the decode's call time.
//   sfp_mfma   back-to-back v_mfma_f32_32x32x16_bf16 on register operands,
//              several independent accumulators per wave; the dense bf16
//              matrix-core rate at the clock the chip holds under load.
//              Every MFMA multiplies the same two operands, so the matrix
//              core's inputs hardly switch between instructions.
//   sfp_mfma_random
//              the same, rotating over four pairs of operands filled with
//              hashed random bf16 values, so consecutive MFMAs multiply
//              unrelated data, as attention on random inputs does: the rate
//              at the clock the chip holds when the operands switch.
// Not part of the attention library: a separate shared object with its own
// C entry points, each enqueued on `stream`; the caller times them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 8;   // 16-byte loads in flight per lane

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  const size_t stride = size_t(gridDim.x) * 256 * kUnroll;
  uint32_t acc = 0;
  for (size_t base = size_t(blockIdx.x) * 256 * kUnroll + threadIdx.x; base < n16; base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * 256;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // one word per work group keeps the loads live
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n16) {
  const size_t stride = size_t(gridDim.x) * 256 * 4;
  for (size_t base = size_t(blockIdx.x) * 256 * 4 + threadIdx.x; base < n16; base += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = base + size_t(u) * 256;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = base + size_t(u) * 256;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

// CH independent 32x32 accumulators per wave: each MFMA depends only on the
// one issued CH steps earlier, so the matrix pipe never waits on a result.
template <int CH>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * float(threadIdx.x + i));
    b[i] = (__bf16)(seed * float(threadIdx.x - i));
  }
  f32x16 c[CH] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = s;
}


// lowbias32 (C. Wellons' integer hash): a well-mixed 32-bit value per input.
__device__ inline uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// As mfma_kernel<8>, with four operand pairs of random values in [-2, 2):
// MFMA j of an iteration multiplies A set j mod 4 by B set (j + 1) mod 4.
__global__ __launch_bounds__(256) void mfma_random_kernel(float* __restrict__ out, int iters, uint32_t seed) {
  constexpr int CH = 8;
  bf16x8 a[4], b[4];
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = hash32(seed ^ hash32(t * 64u + s * 16u + i));
      const uint32_t hb = hash32(seed ^ hash32(t * 64u + s * 16u + 8u + i));
      a[s][i] = (__bf16)(float(ha >> 8) * 0x1p-22f - 2.f);
      b[s][i] = (__bf16)(float(hb >> 8) * 0x1p-22f - 2.f);
    }
  f32x16 c[CH] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + 1) & 3], c[j], 0, 0, 0);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[j][i];
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = sum;
}

// One work group per (head, key range); 16 lanes cover one 256-byte slice, 16
// rows per pass, kUnroll / 2 passes of K and V in flight per lane.
__global__ __launch_bounds__(256) void slices_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                     int rows_per_group, int heads, uint32_t* __restrict__ sink) {
  const int u = blockIdx.x, s = blockIdx.y;
  const int c16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;
  const size_t row16 = size_t(heads) * 16;                 // 16-byte units per row
  u32x4 acc = {0, 0, 0, 0};
  for (int r = 0; r < rows_per_group; r += 16 * (kUnroll / 2)) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll / 2; ++j) {
      const size_t i = (size_t(s) * rows_per_group + r + j * 16 + rsub) * row16 + size_t(u) * 16 + c16;
      x[2 * j] = __builtin_nontemporal_load(k + i);
      x[2 * j + 1] = __builtin_nontemporal_load(v + i);
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= x[j];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[blockIdx.y * gridDim.x + blockIdx.x] = 1;
}

typedef __attribute__((address_space(3))) void lds_void;

// The same bytes by DMA: wave w takes every 4th step of R rows of K and of V
// (NS stages of R * 512 bytes per wave), waits for a stage and reissues it at
// once (no work on the data: the stream alone). Nontemporal policy (aux 2).
// `lds` holds 4 * NS * R * 512 bytes.
template <int NS, int R>
__device__ __forceinline__ void stream_slices(uint8_t* lds, const void* k, const void* v, uint32_t bytes,
                                              int rows_per_group, int heads) {
  constexpr int SB = R * 512, NI = R / 4;
  const int u = blockIdx.x, s = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6), lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(k), (short)0, int(bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(v), (short)0, int(bytes), 0x00020000);
  const uint32_t row_bytes = uint32_t(heads) * 256;
  const int nsteps = rows_per_group / R / 4;
  const uint32_t lane_off = uint32_t(lane / 16) * row_bytes + uint32_t(u) * 256 + uint32_t(lane % 16) * 16;
  uint8_t* ring = lds + wave * NS * SB;
  auto issue = [&](int st, int step) {
    const uint32_t row0 = uint32_t(s * rows_per_group + (step * 4 + wave) * R);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ring + st * SB + i * 1024), 16,
                                               (row0 + 4 * i) * row_bytes + lane_off, 0, 0, 2);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(ring + st * SB + SB / 2 + i * 1024), 16,
                                               (row0 + 4 * i) * row_bytes + lane_off, 0, 0, 2);
  };
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nsteps) issue(st, st);
  for (int step = 0; step < nsteps; ++step) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * 2 * NI) : "memory");
    if (step + NS < nsteps) issue(step % NS, step + NS);
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int NS, int R>
__global__ __launch_bounds__(256) void slices_lds_kernel(const void* k, const void* v, uint32_t bytes,
                                                         int rows_per_group, int heads) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * NS * R * 512];
  stream_slices<NS, R>(lds, k, v, bytes, rows_per_group, heads);
}

// Decode-shaped partials: output row `row` (16 per kv head) of split s holds
// 128 floats at part_o[(row * splits + s) * 128] and (max, sum) at
// part_ml[(row * splits + s) * 2], the decode library's workspace layout.
constexpr int kChainRows = 16;     // query rows per kv head (n * G at batch 1, cross masks)
constexpr int kChainSplitsMax = 32;

// One wave merges one output row the way the decode's combine loads it:
// 32 lanes cover a split's 128 values (4 each), the two halves of the wave
// take alternate splits, every load first; the values are summed (the
// probe times the data movement, not the rescaling).
__device__ __forceinline__ void chain_merge_row(const float* part_o, const float* part_ml, int splits, int row,
                                                uint16_t* out, int lane) {
  const int d4 = lane % 32, cls = lane / 32;
  const float* po = part_o + size_t(row) * splits * 128 + 4 * d4;
  const float* ml = part_ml + size_t(row) * splits * 2;
  float w = lane < splits ? ml[2 * lane] + ml[2 * lane + 1] : 0.f;
  f32x4 xs[kChainSplitsMax / 2];
#pragma unroll
  for (int i = 0; i < kChainSplitsMax / 2; ++i) {
    const int s = cls + 2 * i;
    xs[i] = s < splits ? *reinterpret_cast<const f32x4*>(po + size_t(s) * 128) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kChainSplitsMax / 2; ++i) acc += xs[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], 32);
  if (cls == 0) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[i] * w);
    *reinterpret_cast<bf16x4*>(out + size_t(row) * 128 + 4 * d4) = ov;
  }
}

// Work group (kv head u, split s): the decode's stream of its key range
// (ring of 2 stages of 32 rows per wave), then its partial of 16 rows, stored
// as the decode's split kernel stores it (one float per thread per pass).
// FUSED: the last group of kv head u to finish merges its 16 rows.
template <bool FUSED>
__global__ __launch_bounds__(256) void chain_split_kernel(const void* k, const void* v, uint32_t bytes,
                                                          int rows_per_group, int heads, float* part_o,
                                                          float* part_ml, uint32_t* ticket, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 2 * 32 * 512];
  __shared__ uint32_t last;
  stream_slices<2, 32>(lds, k, v, bytes, rows_per_group, heads);
  const int u = blockIdx.x, s = blockIdx.y, splits = gridDim.y;
  for (int idx = threadIdx.x; idx < kChainRows * 128; idx += 256) {
    const int row = u * kChainRows + idx / 128, d = idx % 128;
    part_o[(size_t(row) * splits + s) * 128 + d] = float(d);
    if (d == 0) {
      part_ml[(size_t(row) * splits + s) * 2 + 0] = 0.f;
      part_ml[(size_t(row) * splits + s) * 2 + 1] = 1.f;
    }
  }
  if constexpr (FUSED) {
    // release this group's partial at device scope, then take a ticket; the
    // group holding the last ticket resets the counter for the next call
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t t = atomicAdd(&ticket[u], 1u);
      last = t == uint32_t(splits - 1);
      if (last) atomicExch(&ticket[u], 0u);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int r = wave; r < kChainRows; r += 4) chain_merge_row(part_o, part_ml, splits, u * kChainRows + r, out, lane);
  }
}

// The library's second kernel: one wave per output row.
__global__ __launch_bounds__(256) void chain_combine_kernel(const float* part_o, const float* part_ml, int splits,
                                                            uint16_t* out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  chain_merge_row(part_o, part_ml, splits, row, out, threadIdx.x & 63);
}
}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `src` with `blocks`
// work groups of 256 threads; writes one word per work group to `sink`
// (blocks words). Returns a hipError_t value (0 on success).
int sfp_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src), bytes / 16,
                     sink);
  return int(hipGetLastError());
}

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned, no overlap).
int sfp_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return int(hipGetLastError());
}

// The decode's read pattern: k and v hold `rows` rows of `heads` * 256 bytes
// each (one bf16 d = 128 row per head); work group (u, s) reads head u's
// slice of rows [s * rows / splits, (s + 1) * rows / splits) of both.
// rows / splits must be a multiple of 64. sink: heads * splits words.
int sfp_read_slices(const void* k, const void* v, int rows, int heads, int splits, uint32_t* sink,
                    hipStream_t stream) {
  if (rows % splits || (rows / splits) % 64) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(slices_kernel, dim3(heads, splits), dim3(256), 0, stream, static_cast<const u32x4*>(k),
                     static_cast<const u32x4*>(v), rows / splits, heads, sink);
  return int(hipGetLastError());
}

// The same by buffer->LDS DMA, ring = 2, 4 or 8 stages per wave (of 32, 16 or
// 8 rows: 128 KiB of LDS per group either way). rows * heads * 256 < 2^31.
int sfp_read_slices_lds(const void* k, const void* v, int rows, int heads, int splits, int ring,
                        hipStream_t stream) {
  const int rpg = rows / splits;
  if (rows % splits || rpg % 128 || size_t(rows) * heads * 256 >= (size_t(1) << 31)) return int(hipErrorInvalidValue);
  const uint32_t bytes = uint32_t(size_t(rows) * heads * 256);
  const dim3 grid(heads, splits);
  if (ring == 2)
    hipLaunchKernelGGL((slices_lds_kernel<2, 32>), grid, dim3(256), 0, stream, k, v, bytes, rpg, heads);
  else if (ring == 4)
    hipLaunchKernelGGL((slices_lds_kernel<4, 16>), grid, dim3(256), 0, stream, k, v, bytes, rpg, heads);
  else if (ring == 8)
    hipLaunchKernelGGL((slices_lds_kernel<8, 8>), grid, dim3(256), 0, stream, k, v, bytes, rpg, heads);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

// The batch-1 decode call's structure with no arithmetic (see the file
// header). k, v: `rows` rows of heads * 256 bytes each, as sfp_read_slices_lds
// (rows / splits a multiple of 128, rows * heads * 256 < 2^31); splits <= 32.
// part: heads * 16 * splits * 130 floats of scratch. out: heads * 16 * 128
// bf16 values. ticket: heads words, zero before the first fused call (each
// fused call leaves them zero). fused = 0: split kernel + combine kernel
// (two launches); fused = 1: one launch.
int sfp_decode_chain(const void* k, const void* v, int rows, int heads, int splits, float* part, uint32_t* ticket,
                     void* out, int fused, hipStream_t stream) {
  if (splits < 1 || splits > kChainSplitsMax || heads < 1 || rows % splits || (rows / splits) % 128 ||
      size_t(rows) * heads * 256 >= (size_t(1) << 31))
    return int(hipErrorInvalidValue);
  const uint32_t bytes = uint32_t(size_t(rows) * heads * 256);
  float* part_o = part;
  float* part_ml = part + size_t(heads) * kChainRows * splits * 128;
  uint16_t* o = static_cast<uint16_t*>(out);
  const dim3 grid(heads, splits);
  if (fused) {
    hipLaunchKernelGGL(chain_split_kernel<true>, grid, dim3(256), 0, stream, k, v, bytes, rows / splits, heads,
                       part_o, part_ml, ticket, o);
  } else {
    hipLaunchKernelGGL(chain_split_kernel<false>, grid, dim3(256), 0, stream, k, v, bytes, rows / splits, heads,
                       part_o, part_ml, ticket, o);
    hipLaunchKernelGGL(chain_combine_kernel, dim3(heads * kChainRows / 4), dim3(256), 0, stream,
                       static_cast<const float*>(part_o), static_cast<const float*>(part_ml), splits, o);
  }
  return int(hipGetLastError());
}

// blocks x 4 waves, each running chains * iters MFMAs of 32x32x16 (32768
// flop each) with chains (4 or 8) independent accumulators; `out` holds
// blocks * 256 floats.
int sfp_mfma(float* out, int blocks, int iters, int chains, hipStream_t stream) {
  if (chains == 8)
    hipLaunchKernelGGL(mfma_kernel<8>, dim3(blocks), dim3(256), 0, stream, out, iters, 1e-3f);
  else
    hipLaunchKernelGGL(mfma_kernel<4>, dim3(blocks), dim3(256), 0, stream, out, iters, 1e-3f);
  return int(hipGetLastError());
}

// blocks x 4 waves, each running 8 * iters MFMAs of 32x32x16 on random
// operands (8 independent accumulators); `out` holds blocks * 256 floats.
int sfp_mfma_random(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_random_kernel, dim3(blocks), dim3(256), 0, stream, out, iters, 0x5eedu);
  return int(hipGetLastError());
}

}  // extern "C"
