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

// ---- buffer loads (gfx950) ----
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Offset that makes a buffer load return zeros (>= every num_records used).
constexpr uint32_t kOobOffset = 0x80000000u;

// Raw buffer resource over `bytes` bytes from `base`: loads at offsets past
// the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes bytes [16 i, 16 i + 16) after `dst` (one contiguous KiB per wave).
// The global address is the buffer base + voff; voff is range-checked
// against the buffer size (past the end: zeros written).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}
// The same with the nontemporal cache policy (`nt`), for data read once and
// not again by this launch (the decode's cache rows): on MI355X it streams a
// strided read of every row's 256-byte head slice about 10% faster at 1 GiB
// and 20% faster at 128 MiB than the default policy. Tiles that other work
// groups re-read from L2 (prefill, backward) keep the default.
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 2);
}

// ---- transposed LDS reads (gfx950) ----
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// Eight ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i % 4 of the 8 bytes that lanes 4e + i / 4 address, as its element
// e (e = 0..3). Written as one asm block that also waits for the results,
// so every output is complete when the statement ends. (Through the
// builtin, the compiler cannot tell which LDS the read touches and waits
// for every buffer->LDS load in flight before it, which would drain a
// prefetch ring on every step.)
__device__ __forceinline__ void tr_read8(u32x2 (&o)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// ---- 32x32x16 MFMA operand order shared by the attention kernels ----
// Row group (4 rows) that MFMA A-operand row group m>>2 reads from a tile of
// 32 rows (keys in the forward). After C = A B^T-style products, accumulator
// register 4g+r of lane half h then holds C row 8g + 4h + r, i.e. tile row
// 4*kSigmaG[2g+h] + r: rows 16h .. 16h+15 of the block, so the accumulator
// registers can feed the next MFMA's B operand (k index = 8h + j) directly.
__device__ __forceinline__ int sigma(int m) {
  constexpr uint32_t kSigmaG = 0x63417250u;  // m>>2 = 0..7 -> 0 5 2 7 1 4 3 6 (nibbles, lowest first)
  return 4 * int((kSigmaG >> (4 * (m >> 2))) & 7u) + (m & 3);
}
// Mask word of a lane whose admitted keys in a 64-key tile are the offsets
// lo..hi: bit 16 kb + 4 g + r is set when the key of score register 4 g + r
// of key block kb, offset 32 kb + reg_key_offset(g, hh) + r, is admitted.
// Those offsets come in runs of 4, so the word is the 64-bit run mask with
// its nibbles permuted: lane half 0 reads nibbles 0 2 1 3 of each 32-key
// block, half 1 nibbles 5 7 4 6.
__device__ __forceinline__ uint32_t tile_mask_word(int lo, int hi, int hh) {
  lo = max(lo, 0);
  hi = min(hi, 63);
  const uint64_t m = hi < lo ? 0ull : (~0ull >> (63 - hi)) & (~0ull << lo);
  uint32_t w = 0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint32_t x = uint32_t(m >> (32 * kb));
    uint32_t o;
    if (hh == 0) {
      o = (x & 0xF00Fu) | ((x >> 4) & 0xF0u) | ((x << 4) & 0xF00u);
    } else {
      const uint32_t y = x >> 16;
      o = ((y >> 4) & 0xFu) | ((y >> 8) & 0xF0u) | ((y & 0xFu) << 8) | ((y << 4) & 0xF000u);
    }
    w |= o << (16 * kb);
  }
  return w;
}

// LDS banks on gfx950: 64 banks of 4 bytes. A 16-byte read (ds_read_b128) is
// served in four passes of 16 lanes: within each half-wave, the lanes whose
// quad index (lane / 4 mod 8) has the same parity; 8-byte reads (ds_read_b64,
// ds_read_b64_tr_b16) in two passes of 32 lanes. A pass in which no two lanes
// hit one bank at different addresses takes one cycle. For rows read in the
// sigma order, a pass covers 4 aligned row quads (sigma groups {0,7,4,3} or
// {5,2,1,6}, plus 8 for the second 32 rows), so with rows of d = 128 bf16
// padded to 320 bytes (rows of one quad then lie 64 bytes apart modulo 256)
// and the 16-byte chunk index XORed with this value of the row quad, the 4
// quads of a pass land in distinct 16-byte slots: the two low bits are
// distinct over each group, and bit 3 (the second 32 rows) is ignored. A
// transposed read (64 bytes from each row of one aligned quad) only sees the
// chunks permuted within those 64 bytes.
__device__ __forceinline__ int row_swizzle128(int quad) { return (quad & 3) ^ ((quad >> 2) & 1); }
// Offset (within a 32-key block) of the 4 keys held in registers 4g..4g+3 by
// lane half h: 16h + 4*(((g&1)*2 + (g>>1)) ^ h).
__device__ __forceinline__ int reg_key_offset(int g, int h) { return 16 * h + 4 * ((((g & 1) * 2 + (g >> 1))) ^ h); }
// Combine a value with the one held by lane l^32 (the other half of the
// wave): v_permlane32_swap exchanges the two halves without going through LDS,
// and the max / sum of the two results is the same whichever half lands where.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


}  // namespace sfa
