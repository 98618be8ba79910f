// Attainable-peak microbenchmarks for MI355X (gfx950), used to state the
// roofline of the attention kernels against what this chip actually reaches
// next to its published figures:
//   sfp_read   streams a device buffer once (16-byte loads, several in flight
//              per lane) and folds it into one word per work group; the
//              bandwidth a read-only kernel such as decode can reach.
//   sfp_copy   copies a buffer (read + write), the pattern of the interleave.
//   sfp_mfma   back-to-back v_mfma_f32_32x32x16_bf16 on register operands,
//              several independent accumulators per wave; the dense bf16
//              matrix-core rate at the clock the chip holds under load.
// Not part of the attention library: a separate shared object with its own
// C entry points, each enqueued on `stream`; the caller times them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

}  // extern "C"
