/*
 * sfattn.h -- C ABI of libsfattn: stream-factorized attention (SFA) on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (Hidden Decoding) expands each of L tokens into n stream
 * representations and runs the unchanged transformer over the expanded
 * sequence of length S = n*L. Stream-factorized attention makes most layers
 * attend within a stream and a few across streams. Sources, cited below by
 * page and section:
 *   [HD-tahou]  "微信WeLM提出Hidden Decoding：大模型推理新范式" (www.tahou.com),
 *               sections 隐式序列缩放的技术细节, 规模化落地的工程优化,
 *               实验效果与成本分析, 中间流的作用验证.
 *   [HD-aiflow] aiflownews.com/?p=965, sections "Latent computation scaling and
 *               Hidden Decoding" and "Tencent's ecosystem first scaling strategy".
 *
 * Conventions shared by every call:
 *   - Indices are 0-based: token i, stream k sits at expanded position
 *     p = i*n + k (the page's 1-based (i-1)n+k, [HD-tahou] 隐式序列缩放的技术细节,
 *     step 1).
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates or frees device memory; decode scratch space is passed in
 *     by the caller (see sf_attn_decode_workspace_bytes), except for
 *     sf_attn_decode_noalloc, whose scratch is a fixed array in the library's
 *     own device memory.
 *   - Calls enqueue work on `stream` (0 = the null stream) and return without
 *     synchronising. Results are valid once the stream has been synchronised.
 *   - Arguments are validated on the host before any HIP call. A rejected call
 *     launches nothing, touches no device state and returns SF_ERR_INVALID
 *     (malformed arguments) or SF_ERR_UNSUPPORTED (well-formed but outside the
 *     supported set). A failed launch returns SF_ERR_DEVICE. In every non-OK
 *     case sf_last_error() describes the problem.
 *   - Calls are re-entrant: the only mutable state is the thread-local error
 *     string (and, for sf_attn_decode_noalloc, the per-GPU scratch array and
 *     the table of its addresses). Calls that write the same output buffer
 *     concurrently race.
 *   - Empty problems (batch == 0 or L == 0) are valid no-ops.
 */
#ifndef SFATTN_H
#define SFATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SF_ABI_VERSION 1

typedef enum {
  SF_OK = 0,
  SF_ERR_INVALID = 1,     /* malformed arguments: null pointer, negative size, T > T_max, ... */
  SF_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported set (head dim, alignment, size limits) */
  SF_ERR_DEVICE = 3       /* the HIP runtime reported an error while launching */
} sf_status;

/* Attention masks of stream-factorized attention ([HD-tahou] 规模化落地的工程优化).
 * For query position p and key position q (both expanded positions):
 *   SF_INTRA        q <= p and q mod n == p mod n: only earlier positions of the
 *                   same stream, itself included (the intra-stream layer).
 *   SF_CROSS_FULL   q <= p: standard causal attention over the expanded sequence
 *                   (the cross-stream layer in its full-attention form; also
 *                   [HD-tahou] 隐式序列缩放的技术细节, step 2).
 *   SF_CROSS_WINDOW q <= p and p - q < window: the cross-stream layer in its
 *                   sliding-window form; `window` counts expanded positions,
 *                   the query itself included. */
typedef enum { SF_INTRA = 0, SF_CROSS_FULL = 1, SF_CROSS_WINDOW = 2 } sf_mode;

/* Returns SF_ABI_VERSION of the loaded library. */
int32_t sf_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next libsfattn call on the same thread. */
const char* sf_last_error(void);

/* Stream interleave ([HD-tahou] 隐式序列缩放的技术细节, step 1: stream k of token
 * i goes to position (i-1)n+k, 1-based) and its exact inverse (used to fill the
 * per-stream KV cache, [HD-aiflow] "Latent computation scaling and Hidden
 * Decoding").
 *   inverse == 0:  dst[b][i*n + k][0:row_bytes] = src[k][b][i][0:row_bytes]
 *                  src layout [n][batch][L][row], dst layout [batch][n*L][row]
 *   inverse == 1:  dst[k][b][i][:] = src[b][i*n + k][:]   (layouts swapped)
 * A row is `row_bytes` opaque bytes (e.g. heads*d*sizeof(element)), so any
 * element type works and the copy is bit-exact. src and dst must not overlap.
 * Any alignment and row size is accepted; 16-byte aligned pointers with
 * row_bytes a multiple of 16 take the widest (fastest) copy.
 * Limits: total bytes / vector width < 2^32 (SF_ERR_UNSUPPORTED otherwise). */
sf_status sf_interleave(const void* src, void* dst, int32_t n, int64_t L, int64_t batch,
                        int64_t row_bytes, int32_t inverse, hipStream_t stream);

/* sf_interleave of `count` tensors of the same n, L and batch in one launch,
 * e.g. Q, K and V of the expansion above (rows of different sizes: hq and
 * hkv heads), or K and V on their way into the per-stream cache. Tensor t is
 * moved exactly as sf_interleave(srcs[t], dsts[t], n, L, batch,
 * row_bytes[t], inverse) would move it; one launch saves the separate
 * launches and ramps of the smaller tensors.
 *   srcs, dsts, row_bytes : HOST arrays of `count` entries; the pointers in
 *                           them are device pointers.
 *   count : 1 .. 4 (SF_ERR_INVALID below 1, SF_ERR_UNSUPPORTED above 4).
 * No destination may overlap any source or another destination
 * (SF_ERR_INVALID). The vector width is the widest that divides every pointer
 * and row size; each tensor must stay below 2^32 such vectors. */
sf_status sf_interleave_multi(const void* const* srcs, void* const* dsts, const int64_t* row_bytes, int32_t count,
                              int32_t n, int64_t L, int64_t batch, int32_t inverse, hipStream_t stream);

/* Expansion of the input: with n copies of the vocabulary embedding, stream
 * k's representation of token i (row ids[b][i] of table k) is placed at
 * expanded position i*n + k ([HD-tahou] 隐式序列缩放的技术细节, step 1, there
 * 1-based as (i-1)n+k). One pass gathers and interleaves:
 *   out[b][i*n + k][:] = tables[k][ids[b][i]][:].
 *   ids    : int32 [batch][L], device.
 *   tables : [n][vocab][row_bytes] bytes (any dtype), device.
 *   out    : [batch][n*L][row_bytes], device; must not overlap the inputs.
 * An id outside [0, vocab) gives a row of zeros. Supported: at most 2^32
 * vectors in out (vectors of 16, 8, 4, 2 or 1 bytes, the widest the row size
 * and the pointers allow); ids 4-byte aligned. */
sf_status sf_expand_embed(const int32_t* ids, const void* tables, void* out, int64_t batch, int32_t n, int64_t L,
                          int64_t vocab, int64_t row_bytes, hipStream_t stream);

/* Rotary position encoding, in place, at continuous expanded positions: row s
 * of the expanded sequence has position pos0 + s ([HD-tahou]
 * 隐式序列缩放的技术细节, step 2: the expanded sequence runs under a
 * continuous position encoding, so a token's streams take consecutive
 * positions). The page does not name the encoding; the rotary encoding in its
 * rotate-half form is used: for j < d/2, with a = (pos0 + s) * base^(-2j/d),
 *   y[j] = x[j] cos a - x[j + d/2] sin a,   y[j + d/2] = x[j + d/2] cos a + x[j] sin a.
 * The angle is formed and reduced in fp64, sin/cos and the rotation in fp32,
 * the result rounded to bf16 once.
 *   x : bf16 [batch][S][heads][d], 8-byte aligned (Q or K before attention).
 * Supported: d a multiple of 8, at most 256; base > 1. */
sf_status sf_rope(void* x, int64_t batch, int64_t S, int32_t heads, int32_t d, float base, int64_t pos0,
                  hipStream_t stream);

/* Prefill attention over the expanded sequence, one of the three masks above,
 * with grouped-query attention ([HD-aiflow] "Tencent's ecosystem first scaling
 * strategy"): query head h reads key/value head h / (hq/hkv).
 *   q, o : bf16 [batch][n*L][hq][d]      (o may not alias q, k or v)
 *   k, v : bf16 [batch][n*L][hkv][d]
 *   lse  : fp32 [batch][hq][n*L] or NULL; lse[b][h][p] = ln sum_{q allowed}
 *          exp(scale * <q_p, k_q>), the natural-log normaliser of row p.
 *   window: used only by SF_CROSS_WINDOW (must be >= 1 there); ignored otherwise.
 *   scale : softmax scale applied to q.k (e.g. 1/sqrt(d)); finite and > 0.
 * Output rows are O[p] = sum_q softmax_q(scale*q_p.k_q over allowed q) v_q,
 * computed with fp32 accumulation and rounded to bf16 once.
 * Supported: d in {64, 128}; hq % hkv == 0; q, k, v, o 16-byte aligned, lse
 * 4-byte aligned; batch*n*L*hq*d <= 2^30 elements. */
sf_status sf_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                      int32_t mode, int64_t window, float scale, hipStream_t stream);

/* Attention for the last stream's queries only: for each token i, the query
 * of stream n-1 at expanded position i*n + n-1 attends to the keys its mode
 * admits there, exactly the rows i*n + n-1 of sf_attn_fwd with the same K, V,
 * mode and window, at about 1/n of the work. Under the cross masks that is
 * every stream's earlier positions; under SF_INTRA stream n-1's own tokens.
 * This is the attention of layers that only the final stream passes through
 * ([HD-tahou] 规模化落地的工程优化: with the KV mirror only the last stream
 * goes through the mirrored layers; 中间流的作用验证: the final stream reads
 * the intermediate streams).
 *   q_last, o_last : bf16 [batch][L][hq][d], row i = stream n-1 of token i.
 *   k, v           : bf16 [batch][n*L][hkv][d], every stream (as sf_attn_fwd).
 *   lse            : fp32 [batch][hq][L] or NULL.
 * Other arguments, errors and the supported set as for sf_attn_fwd, with at
 * most 2^30 elements in q_last and in k. */
sf_status sf_attn_fwd_last_stream(const void* q_last, const void* k, const void* v, void* o_last, float* lse,
                                  int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                                  int32_t mode, int64_t window, float scale, hipStream_t stream);

/* Bytes of device workspace sf_attn_bwd needs (0 if the arguments are invalid
 * or the problem is empty): lse*log2(e) and D = rowsum(dout * o) for every
 * (batch, position, query head), 8 bytes each. */
size_t sf_attn_bwd_workspace_bytes(int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv, int32_t d,
                                   int32_t mode, int64_t window);

/* Backward of sf_attn_fwd: the gradients of the loss sum(dout * o) with
 * respect to q, k and v, for training ([HD-tahou] 实验效果与成本分析 states
 * the method's cost as training step times). With P the masked softmax of
 * scale * q k^T (as in sf_attn_fwd):
 *   dv = P^T dout,  dP = dout v^T,  dS = P * (dP - rowsum(dout * o)),
 *   dq = scale dS k,  dk = scale dS^T q,
 * summed over the query heads of a group for dk and dv.
 *   q, o, dout, dq : bf16 [batch][n*L][hq][d];  k, v, dk, dv : bf16 [batch][n*L][hkv][d].
 *   lse : fp32 [batch][hq][n*L], the natural-log LSE that sf_attn_fwd returned for o.
 *   workspace : at least sf_attn_bwd_workspace_bytes(...) bytes, 16-byte
 *               aligned; contents on entry do not matter.
 * dq, dk, dv are overwritten (not accumulated); they must not overlap each
 * other, the inputs or the workspace. Results are deterministic (no
 * atomics). Other arguments, errors and the supported set as for
 * sf_attn_fwd. */
sf_status sf_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int64_t batch, int32_t n, int64_t L, int32_t hq, int32_t hkv,
                      int32_t d, int32_t mode, int64_t window, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Bytes of device workspace sf_attn_decode needs for these arguments (0 if the
 * arguments are invalid or the problem is empty). num_splits as for
 * sf_attn_decode; the result depends on nothing else. */
size_t sf_attn_decode_workspace_bytes(int64_t batch, int32_t n, int64_t T, int32_t hq,
                                      int32_t hkv, int32_t d, int32_t mode, int64_t window,
                                      int32_t num_splits);

/* One decode step: the n stream queries of the newest token t = T-1 in one
 * pass ([HD-tahou] 实验效果与成本分析: the n streams of a token go through one
 * forward pass in parallel) against a per-stream KV cache ([HD-aiflow] "Latent
 * computation scaling and Hidden Decoding"; independent per-stream state,
 * [HD-tahou] 中间流的作用验证).
 *   q_new, o_new : bf16 [batch][n][hq][d]; row k is stream k of token T-1,
 *                  i.e. expanded position (T-1)*n + k.
 *   k_cache, v_cache : bf16 [batch][n][T_max][hkv][d]; tokens 0..T-1 are valid
 *                  and the caller has already written token T-1's n rows.
 *   The result equals rows (T-1)*n .. (T-1)*n + n-1 of sf_attn_fwd over the T
 *   tokens with the same mode and window: under the cross masks stream k of
 *   the new token also sees streams 0..k of that token; under SF_INTRA it sees
 *   tokens 0..T-1 of its own stream only.
 *   workspace : device scratch of at least sf_attn_decode_workspace_bytes(...)
 *               bytes, 16-byte aligned; may be NULL when that size is 0 (one
 *               split). Its contents on entry do not matter.
 *   num_splits: how many pieces each key range is cut into (0 = chosen by the
 *               library from the problem size; at most 1024 are used). The
 *               result does not depend on it beyond float rounding.
 * Supported: d in {64, 128}; hq % hkv == 0; n*G <= 64 query rows per key/value
 * head under the cross masks (G = hq/hkv), G <= 64 under SF_INTRA; 16-byte
 * aligned q_new, caches and o_new; T_max*hkv*d*2 < 2^31 (bytes of one
 * stream's cache of one batch element). */
sf_status sf_attn_decode(const void* q_new, const void* k_cache, const void* v_cache, void* o_new,
                         int64_t batch, int32_t n, int64_t T, int64_t T_max, int32_t hq,
                         int32_t hkv, int32_t d, int32_t mode, int64_t window, float scale,
                         int32_t num_splits, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of decode scratch that sf_attn_decode_noalloc holds per GPU. */
#define SF_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/* sf_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It computes exactly what sf_attn_decode
 * computes (same kernels and split plan, bitwise equal results), with the
 * split partials in a fixed device array of SF_DECODE_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends. It calls no
 * hipMalloc, hipFree or other allocating routine.
 *   Arguments, supported set and errors as for sf_attn_decode, and
 *   SF_ERR_UNSUPPORTED when the plan's workspace
 *   (sf_attn_decode_workspace_bytes with the same arguments) exceeds
 *   SF_DECODE_SCRATCH_BYTES. Every plan with num_splits = 0 fits; a large
 *   explicit num_splits may not.
 *   Every call on one GPU shares that GPU's array, and nothing in it needs
 *   to start at zero. Calls that overlap in time on one GPU (for example on
 *   two streams) race on the array and must not be issued. */
sf_status sf_attn_decode_noalloc(const void* q_new, const void* k_cache, const void* v_cache, void* o_new,
                                 int64_t batch, int32_t n, int64_t T, int64_t T_max, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t mode, int64_t window, float scale,
                                 int32_t num_splits, hipStream_t stream);

/* Bytes of device workspace sf_attn_decode_paged needs (0 if the arguments
 * are invalid or the problem is empty); max_T and num_splits as there. */
size_t sf_attn_decode_paged_workspace_bytes(int64_t batch, int32_t n, int64_t max_T, int32_t hq,
                                            int32_t hkv, int32_t d, int32_t mode, int64_t window,
                                            int32_t num_splits);

/* sf_attn_decode for a batch of sequences of different lengths whose
 * per-stream caches are spread over fixed-size pages. For serving: the
 * production decode the pages describe ([HD-tahou] 实验效果与成本分析, decode
 * at small batch is bound by memory bandwidth) runs many sequences of
 * different lengths at once.
 *   q_new, o_new : bf16 [batch][n][hq][d]; row k of sequence b is stream k of
 *                  its newest token T_b - 1 (expanded position (T_b-1)*n + k).
 *   k_pages, v_pages : bf16 page pools [num_pages][page_size][hkv][d].
 *   block_table : int32 [batch][n][max_pages], device: token t of stream k of
 *                  sequence b is row t mod page_size of page
 *                  block_table[b][k][t / page_size]. Only the entries of pages
 *                  below T_b are read; an entry outside [0, num_pages) is read
 *                  as a page of zeros (nothing outside the pools is touched).
 *   seq_lens : int32 [batch], device: T_b, the tokens in sequence b's cache,
 *              token T_b - 1's n rows already written. A value outside
 *              [1, max_T] makes that sequence's output rows NaN.
 *   max_T : an upper bound of every T_b, known on the host; it sizes the
 *           split plan and the workspace (with SF_CROSS_WINDOW only the last
 *           window positions count, so a large max_T costs nothing there).
 * Each sequence's result equals sf_attn_decode over its own T_b tokens with
 * the cache gathered from its pages.
 * Supported: as sf_attn_decode, plus page_size a multiple of 32 tokens,
 * max_pages * page_size >= max_T, page_size*hkv*d*2 < 2^31 and
 * n*max_T < 2^31; block_table and seq_lens 4-byte aligned. */
sf_status sf_attn_decode_paged(const void* q_new, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seq_lens, void* o_new,
                               int64_t batch, int32_t n, int64_t max_T, int64_t num_pages,
                               int32_t page_size, int64_t max_pages, int32_t hq, int32_t hkv, int32_t d,
                               int32_t mode, int64_t window, float scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SFATTN_H */
