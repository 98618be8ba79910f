// C ABI of libsfattn: host-side validation, then dispatch to the launchers.
//
// Every check runs before any HIP call, so a rejected call has no device
// side effects (and the checks can be exercised on a machine without a GPU).
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/sfattn.h"
#include "launch.h"

namespace {

thread_local std::string g_error;

sf_status fail(sf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

sf_status ok() {
  g_error.clear();
  return SF_OK;
}

sf_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SF_ERR_DEVICE, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
}

// a*b*... without overflow; false if the product exceeds INT64_MAX.
bool mul_ok(int64_t& acc, int64_t x) {
  int64_t r;
  if (__builtin_mul_overflow(acc, x, &r)) return false;
  acc = r;
  return true;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + uint64_t(bbytes) && b0 < a0 + uint64_t(abytes);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

const char* mode_name(int32_t m) {
  switch (m) {
    case SF_INTRA: return "intra";
    case SF_CROSS_FULL: return "cross_full";
    case SF_CROSS_WINDOW: return "cross_window";
    default: return "?";
  }
}

// Checks shared by prefill and decode.
sf_status check_heads(int32_t n, int32_t hq, int32_t hkv, int32_t d, int32_t mode, int64_t window,
                      float scale) {
  if (n < 1) return fail(SF_ERR_INVALID, "n must be >= 1 (got %d)", n);
  if (hq < 1 || hkv < 1) return fail(SF_ERR_INVALID, "head counts must be >= 1 (hq=%d hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(SF_ERR_INVALID, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (mode != SF_INTRA && mode != SF_CROSS_FULL && mode != SF_CROSS_WINDOW)
    return fail(SF_ERR_INVALID, "unknown mode %d", mode);
  if (mode == SF_CROSS_WINDOW && window < 1)
    return fail(SF_ERR_INVALID, "cross_window needs window >= 1 (got %lld)", (long long)window);
  if (!std::isfinite(scale)) return fail(SF_ERR_INVALID, "scale must be finite");
  if (!(scale > 0.0f)) return fail(SF_ERR_UNSUPPORTED, "scale must be > 0 (got %g)", double(scale));
  if (d != 64 && d != 128) return fail(SF_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  return SF_OK;
}

// Validation shared by sf_attn_decode and sf_attn_decode_noalloc: everything
// but the workspace. On SF_OK with batch > 0, `plan` holds the launch plan.
sf_status check_decode(const void* q_new, const void* k_cache, const void* v_cache, const void* o_new,
                       int64_t batch, int32_t n, int64_t T, int64_t T_max, int32_t hq, int32_t hkv, int32_t d,
                       int32_t mode, int64_t window, float scale, int32_t num_splits, sfa::DecodePlan& plan) {
  if (batch < 0) return fail(SF_ERR_INVALID, "batch must be >= 0");
  if (T < 1) return fail(SF_ERR_INVALID, "T must be >= 1 (got %lld)", (long long)T);
  if (T_max < T) return fail(SF_ERR_INVALID, "T (%lld) exceeds T_max (%lld)", (long long)T, (long long)T_max);
  if (num_splits < 0) return fail(SF_ERR_INVALID, "num_splits must be >= 0");
  sf_status st = check_heads(n, hq, hkv, d, mode, window, scale);
  if (st != SF_OK) return st;
  const int32_t G = hq / hkv;
  if (mode == SF_INTRA ? G > 64 : int64_t(n) * G > 64)
    return fail(SF_ERR_UNSUPPORTED, "%s decode supports at most 64 query rows per kv head (n=%d, G=%d)",
                mode_name(mode), n, G);
  if (batch == 0) return ok();
  if (!q_new || !k_cache || !v_cache || !o_new) return fail(SF_ERR_INVALID, "null q_new, cache or o_new");
  int64_t ce = batch, qe = batch;
  if (!mul_ok(ce, n) || !mul_ok(ce, T_max) || !mul_ok(ce, hkv) || !mul_ok(ce, d) || !mul_ok(qe, n) ||
      !mul_ok(qe, hq) || !mul_ok(qe, d))
    return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (!aligned(q_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o_new, 16))
    return fail(SF_ERR_UNSUPPORTED, "q_new, caches and o_new must be 16-byte aligned");
  if (overlaps(o_new, qe * 2, q_new, qe * 2) || overlaps(o_new, qe * 2, k_cache, ce * 2) ||
      overlaps(o_new, qe * 2, v_cache, ce * 2))
    return fail(SF_ERR_INVALID, "o_new overlaps an input");
  if (ce > (int64_t(1) << 40) || T_max * hkv * d * 2 > INT32_MAX)
    return fail(SF_ERR_UNSUPPORTED, "cache too large (T_max * hkv * d * 2 = %lld bytes per stream, at most 2^31 - 1)",
                (long long)(T_max * hkv * d * 2));
  plan = sfa::plan_decode(batch, n, T, hq, hkv, d, mode, window, num_splits);
  if (plan.units > 65535)
    return fail(SF_ERR_UNSUPPORTED, "decode supports at most 65535 key ranges (batch*hkv%s = %lld)",
                mode == SF_INTRA ? "*n" : "", (long long)plan.units);
  return SF_OK;
}

// Decode scratch of sf_attn_decode_noalloc: one fixed array in device memory
// per GPU, held until the process ends. Host code never uses the array's name
// as an address (on the host it names a stand-in, not device memory): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept in `g_scratch`.
__device__ __align__(256) unsigned char scratch[SF_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

sf_status decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SF_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return device_status(e == hipSuccess ? hipErrorInvalidSymbol : e,
                                                      "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SF_OK;
}

}  // namespace

extern "C" {

int32_t sf_abi_version(void) { return SF_ABI_VERSION; }

const char* sf_last_error(void) { return g_error.c_str(); }

sf_status sf_interleave(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                        int64_t row_bytes, int32_t inverse, hipStream_t stream) {
  if (n < 1) return fail(SF_ERR_INVALID, "n must be >= 1 (got %d)", n);
  if (L < 0 || batch < 0) return fail(SF_ERR_INVALID, "L and batch must be >= 0");
  if (row_bytes < 1) return fail(SF_ERR_INVALID, "row_bytes must be >= 1");
  if (inverse != 0 && inverse != 1) return fail(SF_ERR_INVALID, "inverse must be 0 or 1");
  if (L == 0 || batch == 0) return ok();
  if (!src || !dst) return fail(SF_ERR_INVALID, "null src or dst");
  int64_t bytes = row_bytes;
  if (!mul_ok(bytes, n) || !mul_ok(bytes, L) || !mul_ok(bytes, batch))
    return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (overlaps(src, bytes, dst, bytes)) return fail(SF_ERR_INVALID, "src and dst overlap");
  const uint64_t align = uint64_t(reinterpret_cast<uintptr_t>(src)) |
                         uint64_t(reinterpret_cast<uintptr_t>(dst)) | uint64_t(row_bytes);
  const int vb = (align & 15) == 0 ? 16 : (align & 7) == 0 ? 8 : (align & 3) == 0 ? 4 : (align & 1) == 0 ? 2 : 1;
  if (uint64_t(bytes) / uint64_t(vb) >= (uint64_t(1) << 32))
    return fail(SF_ERR_UNSUPPORTED, "interleave of %lld bytes exceeds 2^32 vectors of %d bytes",
                (long long)bytes, vb);
  return device_status(sfa::launch_interleave(src, dst, n, L, batch, row_bytes, inverse, stream),
                       "sf_interleave launch");
}

sf_status sf_interleave_multi(const void* const* srcs, void* const* dsts, const int64_t* row_bytes, int32_t count,
                              int32_t n, int64_t L, int64_t batch, int32_t inverse, hipStream_t stream) {
  if (count < 1) return fail(SF_ERR_INVALID, "count must be >= 1 (got %d)", count);
  if (count > sfa::kMaxInterleave)
    return fail(SF_ERR_UNSUPPORTED, "at most %d tensors per call (got %d)", sfa::kMaxInterleave, count);
  if (!srcs || !dsts || !row_bytes) return fail(SF_ERR_INVALID, "null srcs, dsts or row_bytes array");
  if (n < 1) return fail(SF_ERR_INVALID, "n must be >= 1 (got %d)", n);
  if (L < 0 || batch < 0) return fail(SF_ERR_INVALID, "L and batch must be >= 0");
  if (inverse != 0 && inverse != 1) return fail(SF_ERR_INVALID, "inverse must be 0 or 1");
  for (int t = 0; t < count; ++t)
    if (row_bytes[t] < 1) return fail(SF_ERR_INVALID, "row_bytes[%d] must be >= 1", t);
  if (L == 0 || batch == 0) return ok();
  int64_t bytes[sfa::kMaxInterleave];
  for (int t = 0; t < count; ++t) {
    if (!srcs[t] || !dsts[t]) return fail(SF_ERR_INVALID, "null src or dst of tensor %d", t);
    bytes[t] = row_bytes[t];
    if (!mul_ok(bytes[t], n) || !mul_ok(bytes[t], L) || !mul_ok(bytes[t], batch))
      return fail(SF_ERR_INVALID, "size of tensor %d overflows int64", t);
  }
  // every destination is disjoint from every source and from the other destinations
  for (int t = 0; t < count; ++t)
    for (int u = 0; u < count; ++u) {
      if (overlaps(dsts[t], bytes[t], srcs[u], bytes[u]))
        return fail(SF_ERR_INVALID, "dst of tensor %d overlaps src of tensor %d", t, u);
      if (u != t && overlaps(dsts[t], bytes[t], dsts[u], bytes[u]))
        return fail(SF_ERR_INVALID, "dsts of tensors %d and %d overlap", t, u);
    }
  const int vb = sfa::interleave_vector_bytes(srcs, dsts, row_bytes, count);
  for (int t = 0; t < count; ++t)
    if (uint64_t(bytes[t]) / uint64_t(vb) >= (uint64_t(1) << 32))
      return fail(SF_ERR_UNSUPPORTED, "tensor %d: %lld bytes exceed 2^32 vectors of %d bytes", t,
                  (long long)bytes[t], vb);
  return device_status(sfa::launch_interleave_multi(srcs, dsts, row_bytes, count, n, L, batch, inverse, stream),
                       "sf_interleave_multi launch");
}

sf_status sf_expand_embed(const int32_t* ids, const void* tables, void* out, int64_t batch, int32_t n, int64_t L,
                          int64_t vocab, int64_t row_bytes, hipStream_t stream) {
  if (n < 1) return fail(SF_ERR_INVALID, "n must be >= 1 (got %d)", n);
  if (L < 0 || batch < 0) return fail(SF_ERR_INVALID, "L and batch must be >= 0");
  if (vocab < 1) return fail(SF_ERR_INVALID, "vocab must be >= 1");
  if (row_bytes < 1) return fail(SF_ERR_INVALID, "row_bytes must be >= 1");
  if (L == 0 || batch == 0) return ok();
  if (!ids || !tables || !out) return fail(SF_ERR_INVALID, "null ids, tables or out");
  int64_t ob = row_bytes, tb = row_bytes, ib = batch;
  if (!mul_ok(ob, n) || !mul_ok(ob, L) || !mul_ok(ob, batch) || !mul_ok(tb, n) || !mul_ok(tb, vocab) ||
      !mul_ok(ib, L) || !mul_ok(ib, 4))
    return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (overlaps(out, ob, tables, tb) || overlaps(out, ob, ids, ib)) return fail(SF_ERR_INVALID, "out overlaps an input");
  if (!aligned(ids, 4)) return fail(SF_ERR_UNSUPPORTED, "ids must be 4-byte aligned");
  const uint64_t align = uint64_t(reinterpret_cast<uintptr_t>(tables)) | uint64_t(reinterpret_cast<uintptr_t>(out)) |
                         uint64_t(row_bytes);
  const int vb = (align & 15) == 0 ? 16 : (align & 7) == 0 ? 8 : (align & 3) == 0 ? 4 : (align & 1) == 0 ? 2 : 1;
  if (uint64_t(ob) / uint64_t(vb) >= (uint64_t(1) << 32) || uint64_t(n) * uint64_t(L) >= (uint64_t(1) << 32) ||
      row_bytes / vb >= (int64_t(1) << 32))
    return fail(SF_ERR_UNSUPPORTED, "expand_embed output of %lld bytes exceeds 2^32 vectors of %d bytes",
                (long long)ob, vb);
  return device_status(sfa::launch_expand_embed(ids, tables, out, batch, n, L, vocab, row_bytes, vb, stream),
                       "sf_expand_embed launch");
}

sf_status sf_rope(void* x, int64_t batch, int64_t S, int32_t heads, int32_t d, float base, int64_t pos0,
                  hipStream_t stream) {
  if (batch < 0 || S < 0) return fail(SF_ERR_INVALID, "batch and S must be >= 0");
  if (heads < 1) return fail(SF_ERR_INVALID, "heads must be >= 1");
  if (d < 2 || d % 2) return fail(SF_ERR_INVALID, "d must be even and >= 2 (got %d)", d);
  if (!(std::isfinite(base) && base > 1.0f)) return fail(SF_ERR_INVALID, "base must be finite and > 1");
  if (pos0 < 0) return fail(SF_ERR_INVALID, "pos0 must be >= 0");
  if (d % 8 || d > 256) return fail(SF_ERR_UNSUPPORTED, "d must be a multiple of 8 and at most 256 (got %d)", d);
  if (batch == 0 || S == 0) return ok();
  if (!x) return fail(SF_ERR_INVALID, "null x");
  int64_t th = batch;
  if (!mul_ok(th, S) || !mul_ok(th, heads) || !mul_ok(th, d / 8)) return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (th >= (int64_t(1) << 32) || S >= (int64_t(1) << 32) || pos0 + S > (int64_t(1) << 40))
    return fail(SF_ERR_UNSUPPORTED, "rope problem too large");
  if (!aligned(x, 8)) return fail(SF_ERR_UNSUPPORTED, "x must be 8-byte aligned");
  return device_status(sfa::launch_rope(x, batch, S, heads, d, double(base), pos0, stream), "sf_rope launch");
}

}  // extern "C"

namespace {

// sf_attn_fwd and sf_attn_fwd_last_stream: the same checks, with q, o and lse
// holding every position (n*L rows) or one row per token (L rows).
sf_status attn_fwd_checked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch,
                           int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d, int32_t mode,
                           int64_t window, float scale, bool last_stream, hipStream_t stream) {
  const char* fn = last_stream ? "sf_attn_fwd_last_stream" : "sf_attn_fwd";
  if (batch < 0 || L < 0) return fail(SF_ERR_INVALID, "batch and L must be >= 0");
  sf_status st = check_heads(n, hq, hkv, d, mode, window, scale);
  if (st != SF_OK) return st;
  if (batch == 0 || L == 0) return ok();
  if (!q || !k || !v || !o) return fail(SF_ERR_INVALID, "null q, k, v or o");
  const int32_t qrows = last_stream ? 1 : n;   // query rows per token
  int64_t qe = batch, kve = batch;
  if (!mul_ok(qe, qrows) || !mul_ok(qe, L) || !mul_ok(qe, hq) || !mul_ok(qe, d) ||
      !mul_ok(kve, n) || !mul_ok(kve, L) || !mul_ok(kve, hkv) || !mul_ok(kve, d))
    return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (qe > (int64_t(1) << 30) || kve > (int64_t(1) << 30))
    return fail(SF_ERR_UNSUPPORTED, "q has %lld and k %lld elements; at most 2^30 each supported", (long long)qe,
                (long long)kve);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SF_ERR_UNSUPPORTED, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(SF_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
  if (overlaps(o, qe * 2, q, qe * 2) || overlaps(o, qe * 2, k, kve * 2) || overlaps(o, qe * 2, v, kve * 2))
    return fail(SF_ERR_INVALID, "o overlaps an input");
  if (lse) {
    const int64_t le = qe / d;   // batch * rows * hq
    if (overlaps(lse, le * 4, o, qe * 2) || overlaps(lse, le * 4, q, qe * 2) ||
        overlaps(lse, le * 4, k, kve * 2) || overlaps(lse, le * 4, v, kve * 2))
      return fail(SF_ERR_INVALID, "lse overlaps another tensor");
  }
  sfa::FwdArgs a{q, k, v, o, lse, batch, n, L, hq, hkv, d, mode, window, scale, last_stream};
  char what[64];
  snprintf(what, sizeof what, "%s launch", fn);
  return device_status(sfa::launch_attn_fwd(a, stream), what);
}

}  // namespace

extern "C" {

sf_status sf_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                      int32_t mode, int64_t window, float scale, hipStream_t stream) {
  return attn_fwd_checked(q, k, v, o, lse, batch, n, L, hq, hkv, d, mode, window, scale, false, stream);
}

sf_status sf_attn_fwd_last_stream(const void* q_last, const void* k, const void* v, void* o_last, float* lse,
                                  int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                                  int32_t mode, int64_t window, float scale, hipStream_t stream) {
  return attn_fwd_checked(q_last, k, v, o_last, lse, batch, n, L, hq, hkv, d, mode, window, scale, true, stream);
}

size_t sf_attn_bwd_workspace_bytes(int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                                   int32_t mode, int64_t window) {
  if (batch <= 0 || L <= 0) return 0;
  if (check_heads(n, hq, hkv, d, mode, window, 1.0f) != SF_OK) return 0;
  return sfa::attn_bwd_workspace_bytes(batch, n, L, hq, mode);
}

sf_status sf_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv,
                      int32_t d, int32_t mode, int64_t window, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (batch < 0 || L < 0) return fail(SF_ERR_INVALID, "batch and L must be >= 0");
  sf_status st = check_heads(n, hq, hkv, d, mode, window, scale);
  if (st != SF_OK) return st;
  if (batch == 0 || L == 0) return ok();
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(SF_ERR_INVALID, "null tensor pointer");
  int64_t qe = batch, kve = batch;
  if (!mul_ok(qe, n) || !mul_ok(qe, L) || !mul_ok(qe, hq) || !mul_ok(qe, d) || !mul_ok(kve, n) ||
      !mul_ok(kve, L) || !mul_ok(kve, hkv) || !mul_ok(kve, d))
    return fail(SF_ERR_INVALID, "tensor size overflows int64");
  if (qe > (int64_t(1) << 30))
    return fail(SF_ERR_UNSUPPORTED, "q has %lld elements; at most 2^30 supported", (long long)qe);
  for (const void* ptr : {q, k, v, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
    if (!aligned(ptr, 16)) return fail(SF_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(SF_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
  const int64_t le = qe / d * 4;   // lse bytes
  const void* outs[3] = {dq, dk, dv};
  const int64_t out_bytes[3] = {qe * 2, kve * 2, kve * 2};
  const void* ins[6] = {q, k, v, o, dout, lse};
  const int64_t in_bytes[6] = {qe * 2, kve * 2, kve * 2, qe * 2, qe * 2, le};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return fail(SF_ERR_INVALID, "an output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return fail(SF_ERR_INVALID, "outputs overlap");
  }
  const size_t need = sfa::attn_bwd_workspace_bytes(batch, n, L, hq, mode);
  if (!workspace || workspace_bytes < need)
    return fail(SF_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(SF_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (overlaps(workspace, int64_t(need), outs[i], out_bytes[i])) return fail(SF_ERR_INVALID, "workspace overlaps a tensor");
  for (int j = 0; j < 6; ++j)
    if (overlaps(workspace, int64_t(need), ins[j], in_bytes[j])) return fail(SF_ERR_INVALID, "workspace overlaps a tensor");
  sfa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, batch, n, L, hq, hkv, d, mode, window, scale, workspace};
  return device_status(sfa::launch_attn_bwd(a, stream), "sf_attn_bwd launch");
}

size_t sf_attn_decode_workspace_bytes(int64_t batch, int32_t n, int64_t T, int32_t hq,
                                      int32_t hkv, int32_t d, int32_t mode, int64_t window,
                                      int32_t num_splits) {
  if (batch <= 0 || T < 1 || num_splits < 0) return 0;
  if (check_heads(n, hq, hkv, d, mode, window, 1.0f) != SF_OK) return 0;
  return sfa::plan_decode(batch, n, T, hq, hkv, d, mode, window, num_splits).ws_bytes;
}

sf_status sf_attn_decode(const void* q_new, const void* k_cache, const void* v_cache, void* o_new,
                         int64_t batch, int32_t n, int64_t T, int64_t T_max, int32_t hq,
                         int32_t hkv, int32_t d, int32_t mode, int64_t window, float scale,
                         int32_t num_splits, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  sfa::DecodePlan plan;
  sf_status st = check_decode(q_new, k_cache, v_cache, o_new, batch, n, T, T_max, hq, hkv, d, mode, window, scale,
                              num_splits, plan);
  if (st != SF_OK || batch == 0) return st;
  const int64_t ce = batch * n * T_max * hkv * d, qe = batch * n * hq * d;
  if ((plan.ws_bytes > 0 && !workspace) || workspace_bytes < plan.ws_bytes)
    return fail(SF_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                plan.ws_bytes);
  if (plan.ws_bytes > 0 && !aligned(workspace, 16))
    return fail(SF_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (overlaps(workspace, int64_t(plan.ws_bytes), o_new, qe * 2) ||
      overlaps(workspace, int64_t(plan.ws_bytes), q_new, qe * 2) ||
      overlaps(workspace, int64_t(plan.ws_bytes), k_cache, ce * 2) ||
      overlaps(workspace, int64_t(plan.ws_bytes), v_cache, ce * 2))
    return fail(SF_ERR_INVALID, "workspace overlaps a tensor");
  sfa::DecodeArgs a{q_new, k_cache, v_cache, o_new, batch, n, T, T_max, hq, hkv, d, mode,
                    window, scale, num_splits, workspace};
  return device_status(sfa::launch_attn_decode(a, plan, stream), "sf_attn_decode launch");
}

sf_status sf_attn_decode_noalloc(const void* q_new, const void* k_cache, const void* v_cache, void* o_new,
                                 int64_t batch, int32_t n, int64_t T, int64_t T_max, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t mode, int64_t window, float scale,
                                 int32_t num_splits, hipStream_t stream) {
  sfa::DecodePlan plan;
  sf_status st = check_decode(q_new, k_cache, v_cache, o_new, batch, n, T, T_max, hq, hkv, d, mode, window, scale,
                              num_splits, plan);
  if (st != SF_OK || batch == 0) return st;
  if (plan.ws_bytes > SF_DECODE_SCRATCH_BYTES)
    return fail(SF_ERR_UNSUPPORTED,
                "this decode needs %zu bytes of scratch; sf_attn_decode_noalloc holds %zu (use fewer splits, "
                "or sf_attn_decode with a workspace)",
                plan.ws_bytes, size_t(SF_DECODE_SCRATCH_BYTES));
  void* scratch = nullptr;
  if (plan.ws_bytes > 0) {
    st = decode_scratch(&scratch);
    if (st != SF_OK) return st;
  }
  sfa::DecodeArgs a{q_new, k_cache, v_cache, o_new, batch, n, T, T_max, hq, hkv, d, mode,
                    window, scale, num_splits, scratch};
  return device_status(sfa::launch_attn_decode(a, plan, stream), "sf_attn_decode_noalloc launch");
}

size_t sf_attn_decode_paged_workspace_bytes(int64_t batch, int32_t n, int64_t max_T, int32_t hq,
                                            int32_t hkv, int32_t d, int32_t mode, int64_t window,
                                            int32_t num_splits) {
  if (batch <= 0 || max_T < 1 || num_splits < 0) return 0;
  if (check_heads(n, hq, hkv, d, mode, window, 1.0f) != SF_OK) return 0;
  return sfa::plan_decode(batch, n, max_T, hq, hkv, d, mode, window, num_splits, true).ws_bytes;
}

sf_status sf_attn_decode_paged(const void* q_new, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seq_lens, void* o_new,
                               int64_t batch, int32_t n, int64_t max_T, int64_t num_pages,
                               int32_t page_size, int64_t max_pages, int32_t hq, int32_t hkv, int32_t d,
                               int32_t mode, int64_t window, float scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch < 0) return fail(SF_ERR_INVALID, "batch must be >= 0");
  if (max_T < 1) return fail(SF_ERR_INVALID, "max_T must be >= 1 (got %lld)", (long long)max_T);
  if (num_pages < 1) return fail(SF_ERR_INVALID, "num_pages must be >= 1");
  if (page_size < 1 || max_pages < 1) return fail(SF_ERR_INVALID, "page_size and max_pages must be >= 1");
  if (page_size % 32)
    return fail(SF_ERR_UNSUPPORTED, "page_size must be a multiple of 32 tokens (got %d)", page_size);
  if (max_pages < (max_T + page_size - 1) / page_size)
    return fail(SF_ERR_INVALID, "max_pages (%lld) x page_size (%d) does not cover max_T (%lld)",
                (long long)max_pages, page_size, (long long)max_T);
  if (num_splits < 0) return fail(SF_ERR_INVALID, "num_splits must be >= 0");
  sf_status st = check_heads(n, hq, hkv, d, mode, window, scale);
  if (st != SF_OK) return st;
  const int32_t G = hq / hkv;
  if (mode == SF_INTRA ? G > 64 : int64_t(n) * G > 64)
    return fail(SF_ERR_UNSUPPORTED, "%s decode supports at most 64 query rows per kv head (n=%d, G=%d)",
                mode_name(mode), n, G);
  if (int64_t(n) * max_T > INT32_MAX)
    return fail(SF_ERR_UNSUPPORTED, "n * max_T must be below 2^31 expanded positions");
  if (int64_t(page_size) * hkv * d * 2 > INT32_MAX)
    return fail(SF_ERR_UNSUPPORTED, "a page must be below 2^31 bytes (page_size * hkv * d * 2)");
  if (batch == 0) return ok();
  if (!q_new || !k_pages || !v_pages || !block_table || !seq_lens || !o_new)
    return fail(SF_ERR_INVALID, "null q_new, page pool, block_table, seq_lens or o_new");
  int64_t pe = num_pages, qe = batch, te = batch;
  if (!mul_ok(pe, page_size) || !mul_ok(pe, hkv) || !mul_ok(pe, d) || !mul_ok(qe, n) || !mul_ok(qe, hq) ||
      !mul_ok(qe, d) || !mul_ok(te, n) || !mul_ok(te, max_pages) || pe > (int64_t(1) << 40))
    return fail(SF_ERR_INVALID, "tensor size overflows");
  if (!aligned(q_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o_new, 16))
    return fail(SF_ERR_UNSUPPORTED, "q_new, page pools and o_new must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(SF_ERR_INVALID, "block_table and seq_lens must be 4-byte aligned");
  if (overlaps(o_new, qe * 2, q_new, qe * 2) || overlaps(o_new, qe * 2, k_pages, pe * 2) ||
      overlaps(o_new, qe * 2, v_pages, pe * 2) || overlaps(o_new, qe * 2, block_table, te * 4) ||
      overlaps(o_new, qe * 2, seq_lens, batch * 4))
    return fail(SF_ERR_INVALID, "o_new overlaps an input");
  const sfa::DecodePlan plan = sfa::plan_decode(batch, n, max_T, hq, hkv, d, mode, window, num_splits, true);
  if (plan.units > 65535)
    return fail(SF_ERR_UNSUPPORTED, "decode supports at most 65535 key ranges (batch*hkv%s = %lld)",
                mode == SF_INTRA ? "*n" : "", (long long)plan.units);
  if ((plan.ws_bytes > 0 && !workspace) || workspace_bytes < plan.ws_bytes)
    return fail(SF_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                plan.ws_bytes);
  if (plan.ws_bytes > 0 && !aligned(workspace, 16))
    return fail(SF_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  const int64_t wb = int64_t(plan.ws_bytes);
  if (overlaps(workspace, wb, o_new, qe * 2) || overlaps(workspace, wb, q_new, qe * 2) ||
      overlaps(workspace, wb, k_pages, pe * 2) || overlaps(workspace, wb, v_pages, pe * 2) ||
      overlaps(workspace, wb, block_table, te * 4) || overlaps(workspace, wb, seq_lens, batch * 4))
    return fail(SF_ERR_INVALID, "workspace overlaps a tensor");
  sfa::DecodeArgs a{q_new, k_pages, v_pages, o_new, batch, n, max_T, max_T, hq, hkv, d, mode,
                    window, scale, num_splits, workspace};
  a.seq_lens = seq_lens;
  a.table = block_table;
  a.page = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  return device_status(sfa::launch_attn_decode(a, plan, stream), "sf_attn_decode_paged launch");
}

}  // extern "C"
