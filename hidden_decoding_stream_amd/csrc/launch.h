// Internal kernel launchers of libsfattn. Arguments arrive here already
// validated by the C ABI layer (api.hip); these functions only pick a
// configuration and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sfa {

hipError_t launch_interleave(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                             int64_t row_bytes, int inverse, hipStream_t stream);
// Up to kMaxInterleave tensors of the same (n, L, batch) in one launch.
constexpr int kMaxInterleave = 4;
hipError_t launch_interleave_multi(const void* const* src, void* const* dst, const int64_t* row_bytes,
                                   int32_t count, int32_t n, int64_t L, int64_t batch, int inverse,
                                   hipStream_t stream);
// Bytes per vector the launch above uses: the widest of 16, 8, 4, 2, 1 that
// divides every pointer and row size.
int interleave_vector_bytes(const void* const* src, void* const* dst, const int64_t* row_bytes, int32_t count);

hipError_t launch_expand_embed(const int32_t* ids, const void* tables, void* out, int64_t batch, int32_t n,
                               int64_t L, int64_t vocab, int64_t row_bytes, int vb, hipStream_t stream);
hipError_t launch_rope(void* x, int64_t batch, int64_t S, int32_t heads, int32_t d, double base, int64_t pos0,
                       hipStream_t stream);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t batch;
  int32_t n;
  int64_t L;
  int32_t hq, hkv, d;
  int32_t mode;
  int64_t window;
  float scale;
  bool last_stream;   // queries: stream n-1 of each token only, q/o [batch][L][hq][d]
};
hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t batch;
  int32_t n;
  int64_t L;
  int32_t hq, hkv, d;
  int32_t mode;
  int64_t window;
  float scale;
  void* ws;
};
size_t attn_bwd_workspace_bytes(int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t mode);
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  void* o;
  int64_t batch;
  int32_t n;
  int64_t T, T_max;
  int32_t hq, hkv, d;
  int32_t mode;
  int64_t window;
  float scale;
  int32_t num_splits;
  void* ws;
  // paged cache: kc/vc are page pools [num_pages][page][hkv][d], T is the
  // largest valid length; null seq_lens means the contiguous cache
  const int32_t* seq_lens = nullptr;
  const int32_t* table = nullptr;
  int32_t page = 0;
  int64_t max_pages = 0, num_pages = 0;
};
// Split plan shared by the workspace query and the launcher.
struct DecodePlan {
  int32_t rows_per_unit;   // query rows that share one key range (n*G cross, G intra)
  int64_t units;           // independent key ranges
  int64_t t_lo;            // first cache token any query may see
  int64_t keys_per_stream; // padded tokens per stream in the key index space
  int64_t keys;            // keys per unit in the key index space (padded)
  int32_t splits;          // pieces per unit
  int64_t chunk;           // keys per piece (multiple of the step)
  size_t ws_bytes;
};
// paged: T is the largest length; the key space then covers any length up to T
DecodePlan plan_decode(int64_t batch, int32_t n, int64_t T, int32_t hq, int32_t hkv, int32_t d,
                       int32_t mode, int64_t window, int32_t num_splits, bool paged = false);
hipError_t launch_attn_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);

}  // namespace sfa
