// Stream interleave and de-interleave (a bit-exact, HBM-bound copy).
//
// Expansion step of Hidden Decoding: stream k of token i is placed at
// expanded position (i-1)n+k, 1-based (page "微信WeLM提出Hidden Decoding：
// 大模型推理新范式", section 隐式序列缩放的技术细节, step 1). 0-based:
//   forward : dst[b][i*n + k][row] = src[k][b][i][row]
//   inverse : dst[k][b][i][row]   = src[b][i*n + k][row]
//
// Each row is row_bytes opaque bytes, moved as VB-byte vectors (VB = 16, 8,
// 4, 2 or 1, the widest that divides the row and both pointers' alignment).
// The work is the flat list of vectors in expanded order, e = row*vpr + v.
// A block of 256 threads takes ILP*256 consecutive vectors; thread t owns
// e = base + t + j*256, so each wave touches 64 consecutive vectors per step
// (coalesced on the expanded side, and on the per-stream side whenever a row
// spans at least a wave's worth of bytes). All loads of a thread are issued
// before its stores. Index math is 32-bit with invariant-divisor division.
#include "common.h"
#include "launch.h"

namespace sfa {

namespace {

constexpr int kThreads = 256;
constexpr int kIlp = 4;

template <int VB> struct Vec;
template <> struct Vec<16> { using T = uint4; };
template <> struct Vec<8> { using T = uint2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

struct InterleaveParams {
  const void* src;
  void* dst;
  uint32_t total;   // vectors in the tensor
  FastDiv vpr;      // vectors per row
  FastDiv S;        // expanded rows per sequence (n*L)
  FastDiv n;        // streams
  uint32_t batch;
  uint32_t L;
  int inverse;
};

template <int VB>
__global__ __launch_bounds__(kThreads) void interleave_kernel(InterleaveParams p) {
  using V = typename Vec<VB>::T;
  const V* __restrict__ src = static_cast<const V*>(p.src);
  V* __restrict__ dst = static_cast<V*>(p.dst);
  const uint32_t base = blockIdx.x * uint32_t(kThreads * kIlp) + threadIdx.x;
  V buf[kIlp];
  uint32_t out_idx[kIlp];
  bool live[kIlp];
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    const uint32_t e = base + uint32_t(j * kThreads);
    live[j] = e < p.total;
    if (!live[j]) continue;
    const uint32_t row = fdiv(e, p.vpr);            // expanded row = b*S + i*n + k
    const uint32_t v = e - row * p.vpr.d;
    const uint32_t b = fdiv(row, p.S);
    const uint32_t pos = row - b * p.S.d;           // i*n + k
    const uint32_t i = fdiv(pos, p.n);
    const uint32_t k = pos - i * p.n.d;
    const uint32_t srow = (k * p.batch + b) * p.L + i;  // per-stream row [k][b][i]
    const uint32_t s_idx = srow * p.vpr.d + v;
    const uint32_t x_idx = e;                           // expanded layout index
    const uint32_t in_idx = p.inverse ? x_idx : s_idx;
    out_idx[j] = p.inverse ? s_idx : x_idx;
    buf[j] = src[in_idx];
  }
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    if (live[j]) dst[out_idx[j]] = buf[j];
  }
}

template <int VB>
hipError_t launch_vb(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                     int64_t row_bytes, int inverse, hipStream_t stream) {
  InterleaveParams p;
  p.src = src;
  p.dst = dst;
  const uint64_t vpr = uint64_t(row_bytes) / VB;
  const uint64_t total = vpr * uint64_t(n) * uint64_t(L) * uint64_t(batch);
  p.total = uint32_t(total);
  p.vpr = make_fastdiv(uint32_t(vpr));
  p.S = make_fastdiv(uint32_t(uint64_t(n) * uint64_t(L)));
  p.n = make_fastdiv(uint32_t(n));
  p.batch = uint32_t(batch);
  p.L = uint32_t(L);
  p.inverse = inverse;
  const uint64_t per_block = uint64_t(kThreads) * kIlp;
  const uint32_t blocks = uint32_t((total + per_block - 1) / per_block);
  hipLaunchKernelGGL(interleave_kernel<VB>, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_interleave(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                             int64_t row_bytes, int inverse, hipStream_t stream) {
  const uint64_t align = uint64_t(reinterpret_cast<uintptr_t>(src)) |
                         uint64_t(reinterpret_cast<uintptr_t>(dst)) | uint64_t(row_bytes);
  if ((align & 15) == 0) return launch_vb<16>(src, dst, n, L, batch, row_bytes, inverse, stream);
  if ((align & 7) == 0) return launch_vb<8>(src, dst, n, L, batch, row_bytes, inverse, stream);
  if ((align & 3) == 0) return launch_vb<4>(src, dst, n, L, batch, row_bytes, inverse, stream);
  if ((align & 1) == 0) return launch_vb<2>(src, dst, n, L, batch, row_bytes, inverse, stream);
  return launch_vb<1>(src, dst, n, L, batch, row_bytes, inverse, stream);
}

}  // namespace sfa
