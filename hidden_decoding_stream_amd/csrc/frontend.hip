// Expansion front-end of Hidden Decoding (HBM-bound, elementwise).
//
// Page "微信WeLM提出Hidden Decoding：大模型推理新范式", section
// 隐式序列缩放的技术细节:
//  step 1 - with n copies of the vocabulary embedding, stream k's
//           representation of token i (row ids[i] of table k) goes to expanded
//           position (i-1)n+k, 1-based: expand_embed_kernel gathers and
//           interleaves in one pass,
//             out[b][i*n + k][:] = tables[k][ids[b][i]][:]   (0-based),
//           with a row of zeros for an id outside [0, vocab);
//  step 2 - the expanded sequence runs under a continuous position encoding:
//           rope_kernel applies rotary encoding (rotate-half form, frequencies
//           base^(-2j/d)) in place at positions pos0 + s of the expanded rows.
//
// expand_embed moves rows as opaque VB-byte vectors (VB = 16..1, the widest
// the row size and pointers allow), like the interleave: each block takes
// 4*256 consecutive output vectors, so both the loads of a table row and the
// stores of the expanded row are coalesced; the output is written with the
// nontemporal cache policy (table rows keep the default: repeated ids re-read
// them). rope, which rewrites its rows in place, keeps the default policy
// (nontemporal there was 25% slower), and forms each angle in fp64
// (position x frequency, reduced modulo 2*pi) and only then takes sin/cos in
// fp32, so large positions keep their accuracy; each thread rotates 4 pairs
// (8-byte loads and stores of bf16).
#include <math.h>

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

struct EmbedParams {
  const int32_t* ids;   // [B][L]
  const void* tables;   // [n][vocab][row]
  void* out;            // [B][n*L][row]
  uint32_t total;       // vectors in out
  FastDiv vpr;          // vectors per row
  FastDiv S;            // n*L
  FastDiv n;
  int32_t L;
  int64_t vocab;
};

template <int VB>
__global__ __launch_bounds__(kThreads) void expand_embed_kernel(EmbedParams p) {
  using T = typename Vec<VB>::T;
  const T* tab = static_cast<const T*>(p.tables);
  T* out = static_cast<T*>(p.out);
  const uint32_t base = blockIdx.x * (kThreads * kIlp) + threadIdx.x;
  T val[kIlp];
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    const uint32_t e = base + j * kThreads;
    val[j] = T{};
    if (e < p.total) {
      const uint32_t row = fdiv(e, p.vpr);
      const uint32_t v = e - row * p.vpr.d;
      const uint32_t b = fdiv(row, p.S);
      const uint32_t pos = row - b * p.S.d;
      const uint32_t i = fdiv(pos, p.n);
      const uint32_t k = pos - i * p.n.d;
      const int32_t id = p.ids[size_t(b) * p.L + i];
      if (id >= 0 && int64_t(id) < p.vocab) val[j] = tab[(size_t(k) * p.vocab + id) * p.vpr.d + v];
    }
  }
#pragma unroll
  for (int j = 0; j < kIlp; ++j) {
    const uint32_t e = base + j * kThreads;
    if (e < p.total) __builtin_nontemporal_store(val[j], out + e);
  }
}

constexpr int kMaxHalf = 128;   // d <= 256

struct RopeParams {
  uint16_t* x;          // [B][S][H][d] bf16, rotated in place
  uint32_t total;       // threads: B*S*H*(d/8)
  FastDiv groups;       // pair groups (of 4) per row and head: d/8
  FastDiv heads;
  FastDiv S;
  int32_t d;
  int64_t pos0;
  double inv_freq[kMaxHalf];   // base^(-2j/d)
};

__global__ __launch_bounds__(kThreads) void rope_kernel(RopeParams p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= p.total) return;
  const uint32_t rh = fdiv(t, p.groups);        // (row, head) index
  const uint32_t grp = t - rh * p.groups.d;
  const uint32_t row = fdiv(rh, p.heads);       // b*S + s
  const uint32_t s = row - fdiv(row, p.S) * p.S.d;
  const int half = p.d / 2;
  const int j0 = 4 * int(grp);
  uint16_t* xr = p.x + size_t(rh) * p.d;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(xr + j0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(xr + half + j0);
  const double pos = double(p.pos0 + int64_t(s));
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  bf16x4 ya, yb;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double ang = pos * p.inv_freq[j0 + q];
    const float r = float(ang - kTwoPi * rint(ang * (1.0 / kTwoPi)));   // in [-pi, pi]
    float sn, cs;
    sincosf(r, &sn, &cs);
    const float xa = float(a[q]), xb = float(b[q]);
    ya[q] = (__bf16)(xa * cs - xb * sn);
    yb[q] = (__bf16)(xb * cs + xa * sn);
  }
  *reinterpret_cast<bf16x4*>(xr + j0) = ya;
  *reinterpret_cast<bf16x4*>(xr + half + j0) = yb;
}

}  // namespace

hipError_t launch_expand_embed(const int32_t* ids, const void* tables, void* out, int64_t batch, int32_t n,
                               int64_t L, int64_t vocab, int64_t row_bytes, int vb, hipStream_t stream) {
  EmbedParams p;
  p.ids = ids;
  p.tables = tables;
  p.out = out;
  const int64_t vpr = row_bytes / vb;
  p.total = uint32_t(batch * n * L * vpr);
  p.vpr = make_fastdiv(uint32_t(vpr));
  p.S = make_fastdiv(uint32_t(n * L));
  p.n = make_fastdiv(uint32_t(n));
  p.L = int32_t(L);
  p.vocab = vocab;
  const dim3 grid((p.total + kThreads * kIlp - 1) / (kThreads * kIlp));
  switch (vb) {
    case 16: hipLaunchKernelGGL(expand_embed_kernel<16>, grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(expand_embed_kernel<8>, grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(expand_embed_kernel<4>, grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(expand_embed_kernel<2>, grid, dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL(expand_embed_kernel<1>, grid, dim3(kThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_rope(void* x, int64_t batch, int64_t S, int32_t heads, int32_t d, double base, int64_t pos0,
                       hipStream_t stream) {
  RopeParams p;
  p.x = static_cast<uint16_t*>(x);
  p.total = uint32_t(batch * S * heads * (d / 8));
  p.groups = make_fastdiv(uint32_t(d / 8));
  p.heads = make_fastdiv(uint32_t(heads));
  p.S = make_fastdiv(uint32_t(S));
  p.d = d;
  p.pos0 = pos0;
  for (int j = 0; j < kMaxHalf; ++j) p.inv_freq[j] = j < d / 2 ? pow(base, -2.0 * j / d) : 0.0;
  const dim3 grid((p.total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(rope_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfa
