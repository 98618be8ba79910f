// Device helpers shared by the libsfattn kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfa {

// Unsigned 32-bit division by a run-time constant d >= 1 with a multiply-high,
// an add and a shift (Granlund & Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, x / d = (mulhi(x, m) + x) >> l for all
// 32-bit x. The add is done in 64 bits so it cannot overflow.
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  f.l = l;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
  uint32_t hi = __umulhi(x, f.m);
  return uint32_t((uint64_t(hi) + x) >> f.l);
}

}  // namespace sfa
