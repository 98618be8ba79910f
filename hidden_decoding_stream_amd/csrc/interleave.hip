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
// before its stores, both with the nontemporal cache policy (every byte is
// read once and written once). Index math is 32-bit with invariant-divisor
// division.
// One launch can move up to kMaxTensors tensors of the same (n, L, batch),
// each with its own row size (Q with hq heads, K and V with hkv): every block
// belongs to one tensor, so small tensors no longer pay a launch and a ramp
// of their own.
#include "common.h"
#include "launch.h"

namespace sfa {

namespace {

constexpr int kThreads = 256;
constexpr int kIlp = 4;

template <int VB> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

struct InterleaveParams {
  const void* src[kMaxInterleave];
  void* dst[kMaxInterleave];
  uint32_t total[kMaxInterleave];    // vectors in tensor t
  FastDiv vpr[kMaxInterleave];       // vectors per row of tensor t
  uint32_t block0[kMaxInterleave];   // first block of tensor t
  int32_t count;
  FastDiv S;        // expanded rows per sequence (n*L)
  FastDiv n;        // streams
  uint32_t batch;
  uint32_t L;
  int inverse;
};

template <int VB>
__global__ __launch_bounds__(kThreads) void interleave_kernel(InterleaveParams p) {
  using V = typename Vec<VB>::T;
  // this block's tensor (wave-uniform), picked by selects rather than by a
  // dynamic index into the parameter arrays
  const uint32_t blk = blockIdx.x;
  const void* src_t = p.src[0];
  void* dst_t = p.dst[0];
  uint32_t total = p.total[0], block0 = 0;
  FastDiv vpr = p.vpr[0];
#pragma unroll
  for (int u = 1; u < kMaxInterleave; ++u) {
    if (u < p.count && blk >= p.block0[u]) {
      src_t = p.src[u];
      dst_t = p.dst[u];
      total = p.total[u];
      vpr = p.vpr[u];
      block0 = p.block0[u];
    }
  }
  const V* __restrict__ src = static_cast<const V*>(src_t);
  V* __restrict__ dst = static_cast<V*>(dst_t);
  const uint32_t base = (blk - block0) * uint32_t(kThreads * kIlp) + threadIdx.x;
  V buf[kIlp];
  uint32_t out_idx[kIlp];
  bool live[kIlp];
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    const uint32_t e = base + uint32_t(j * kThreads);
    live[j] = e < total;
    if (!live[j]) continue;
    const uint32_t row = fdiv(e, vpr);              // expanded row = b*S + i*n + k
    const uint32_t v = e - row * vpr.d;
    const uint32_t b = fdiv(row, p.S);
    const uint32_t pos = row - b * p.S.d;           // i*n + k
    const uint32_t i = fdiv(pos, p.n);
    const uint32_t k = pos - i * p.n.d;
    const uint32_t srow = (k * p.batch + b) * p.L + i;  // per-stream row [k][b][i]
    const uint32_t s_idx = srow * vpr.d + v;
    const uint32_t x_idx = e;                           // expanded layout index
    const uint32_t in_idx = p.inverse ? x_idx : s_idx;
    out_idx[j] = p.inverse ? s_idx : x_idx;
    buf[j] = __builtin_nontemporal_load(src + in_idx);
  }
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    if (live[j]) __builtin_nontemporal_store(buf[j], dst + out_idx[j]);
  }
}

template <int VB>
hipError_t launch_vb(const void* const* src, void* const* dst, const int64_t* row_bytes, int32_t count,
                     int32_t n, int64_t L, int64_t batch, int inverse, hipStream_t stream) {
  InterleaveParams p{};
  const uint64_t per_block = uint64_t(kThreads) * kIlp;
  uint64_t blocks = 0;
  for (int t = 0; t < count; ++t) {
    const uint64_t vpr = uint64_t(row_bytes[t]) / VB;
    const uint64_t total = vpr * uint64_t(n) * uint64_t(L) * uint64_t(batch);
    p.src[t] = src[t];
    p.dst[t] = dst[t];
    p.total[t] = uint32_t(total);
    p.vpr[t] = make_fastdiv(uint32_t(vpr));
    p.block0[t] = uint32_t(blocks);
    blocks += (total + per_block - 1) / per_block;
  }
  p.count = count;
  p.S = make_fastdiv(uint32_t(uint64_t(n) * uint64_t(L)));
  p.n = make_fastdiv(uint32_t(n));
  p.batch = uint32_t(batch);
  p.L = uint32_t(L);
  p.inverse = inverse;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(interleave_kernel<VB>, dim3(uint32_t(blocks)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int interleave_vector_bytes(const void* const* src, void* const* dst, const int64_t* row_bytes, int32_t count) {
  uint64_t align = 0;
  for (int t = 0; t < count; ++t)
    align |= uint64_t(reinterpret_cast<uintptr_t>(src[t])) | uint64_t(reinterpret_cast<uintptr_t>(dst[t])) |
             uint64_t(row_bytes[t]);
  return (align & 15) == 0 ? 16 : (align & 7) == 0 ? 8 : (align & 3) == 0 ? 4 : (align & 1) == 0 ? 2 : 1;
}

hipError_t launch_interleave_multi(const void* const* src, void* const* dst, const int64_t* row_bytes,
                                   int32_t count, int32_t n, int64_t L, int64_t batch, int inverse,
                                   hipStream_t stream) {
  switch (interleave_vector_bytes(src, dst, row_bytes, count)) {
    case 16: return launch_vb<16>(src, dst, row_bytes, count, n, L, batch, inverse, stream);
    case 8: return launch_vb<8>(src, dst, row_bytes, count, n, L, batch, inverse, stream);
    case 4: return launch_vb<4>(src, dst, row_bytes, count, n, L, batch, inverse, stream);
    case 2: return launch_vb<2>(src, dst, row_bytes, count, n, L, batch, inverse, stream);
    default: return launch_vb<1>(src, dst, row_bytes, count, n, L, batch, inverse, stream);
  }
}

hipError_t launch_interleave(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                             int64_t row_bytes, int inverse, hipStream_t stream) {
  void* d = dst;
  return launch_interleave_multi(&src, &d, &row_bytes, 1, n, L, batch, inverse, stream);
}

}  // namespace sfa
