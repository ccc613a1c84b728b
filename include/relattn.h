/*
 * relattn.h -- C ABI of the MI355X (gfx950) relative-attention forward library.
 *
 * The operation (page "SGLang and Miles Add Day-0 Support for Inkling",
 * section "Attention with Relative Positional Embedding"):
 *
 *   rel_logits(t,h,d) = r[t,h,:] . P[:,d]                      for d in [0, E)
 *   l(i,j,h) = s*alpha * q[i,h,:] . k[j,g(h),:]
 *              + [0 <= i-j < E] * s * rel_logits(i,h,i-j)
 *   out[i,h,:] = sum_j softmax_j(l(i,.,h)) * v[j,g(h),:]
 *
 * with keys j > i masked (causal) and, for a sliding-window layer, keys with
 * i-j >= window masked too ("Attention layout" paragraph of that section).
 * s is the length-dependent log-scale on q and on the relative logits; the
 * pages give no formula, this library uses s = max(1, ln(Lseq)/ln(4096)) when
 * log_scale is set and s = 1 otherwise (Lseq = T for prefill, L for decode,
 * seq_len for rel_logits).  GQA: g(h) = h / (Hq/Hkv).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor is caller-owned device memory, row-major and contiguous, with
 *   a 16-byte aligned base address.  Inputs are read only; outputs are fully
 *   overwritten and must not alias an input.
 * - dtype: RA_BF16 or RA_F32 for q, k, v, r, P and out (one dtype per call);
 *   lse and the rel_logits output are always float32.
 * - P is passed distance-major: P_cols[E][d_r] with P_cols[d][c] = P[c][d],
 *   i.e. row d holds the d_r coefficients that r is dotted with for distance d
 *   (the layout of a linear-layer weight mapping d_r features to E outputs).
 *   The pages index P by column, P[:, d]; taking its transpose makes the d_r
 *   coefficients of one distance contiguous, which is what every kernel
 *   reads (one distance per MFMA row), so no call needs a transposed copy.
 * - Supported shapes: D == 128; d_r a multiple of 16 with 16 <= d_r <= 128
 *   (ignored when rel_extent == 0); Hq % Hkv == 0.  Others return
 *   RA_ERR_UNSUPPORTED.  The pages fix no d_r; the bound of 128 is what the
 *   prefill kernel can hold of r in registers as MFMA operands beside q, S
 *   and O at two waves per SIMD.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *   stream) and the call returns without synchronising, copying to the host or
 *   reading device data on the host, so calls can be captured in a hipGraph.
 *   The library allocates no device memory and keeps no per-pointer state;
 *   the one device buffer it holds is the fixed decode scratch of
 *   rel_attn_decode_noalloc (16 MiB per device, from the library's load).
 * - Errors: argument errors are detected on the host before any HIP call and
 *   return a negative code; a failed launch returns RA_ERR_HIP.  In both cases
 *   rel_attn_last_error() returns a message for the calling thread.  The
 *   library never aborts or prints.  A device fault surfaces at the caller's
 *   next synchronisation, as with any HIP kernel.
 * - Results are deterministic: the same inputs give the same bits (no atomics,
 *   fixed reduction orders).
 */
#ifndef RELATTN_H
#define RELATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative or inconsistent size */
  RA_ERR_UNSUPPORTED = -2, /* legal but not implemented (D != 128, d_r outside range, ...) */
  RA_ERR_WORKSPACE = -3,   /* decode workspace missing or smaller than the plan */
  RA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

enum { RA_BF16 = 1, RA_F32 = 2 };

/*
 * Prefill (self-attention over positions 0..T-1 of each sequence).
 *   q   [B, T, Hq, D]       k, v [B, T, Hkv, D]       r [B, T, Hq, d_r]
 *   P_cols [E, d_r]         out [B, T, Hq, D] (dtype)  lse [B, Hq, T] float32 or NULL
 * alpha: the attention scale (e.g. 1/sqrt(D)).  rel_extent E >= 0 (0 = no
 * relative bias; r and P_cols may then be NULL).  window >= 0 (0 = full
 * causal; W >= 1 keeps keys with 0 <= i-j < W).  log_scale: 0 or 1.
 * lse[b,h,i] = natural log of sum_j exp(l(i,j,h)).
 * B == 0 or T == 0 is a no-op that returns RA_OK.
 */
int rel_attn_prefill(const void* q, const void* k, const void* v, const void* r,
                     const void* P_cols, void* out, float* lse, int dtype,
                     int B, int T, int Hq, int Hkv, int D, int d_r,
                     float alpha, int rel_extent, int window, int log_scale,
                     void* stream);

/*
 * Extend: the new rows of several sequences against their KV caches
 * (chunked prefill over a cached prefix, packed variable-length batches,
 * paged caches -- the "extend" kernels of the SGLang page's AMD path).
 * Sequence b holds kv_len[b] tokens in its cache, the last
 * n_b = q_start[b+1] - q_start[b] of which are its new rows: new row t of b
 * (packed row q_start[b] + t) sits at position kv_len[b] - n_b + t and sees
 * the cached keys at positions 0 .. its own under the causal / window mask,
 * with the relative bias by distance as in prefill.  s uses Lseq = kv_len[b]
 * (one scale per sequence, computed on the device in float32).
 *   q [total_q, Hq, D]   r [total_q, Hq, d_r]   P_cols [E, d_r]
 *   out [total_q, Hq, D] (dtype)   lse [Hq, total_q] float32 or NULL
 *   q_start [B+1], kv_len [B]: int32 device arrays (4-byte aligned),
 *     q_start[0] = 0, non-decreasing, q_start[B] = total_q.
 *   Contiguous caches (block_table == NULL): k, v [B, cache_len, Hkv, D].
 *   Paged caches: k, v [num_pages, page_size, Hkv, D]; key j of sequence b
 *     is slot j % page_size of page block_table[b * max_pages + j / page_size]
 *     (int32 device array [B, max_pages]); page_size a positive multiple of
 *     32 (else RA_ERR_UNSUPPORTED).
 *   max_q: a host bound on every n_b; it sizes the launch.
 * The device arrays are not read on the host.  Whatever they hold, every
 * access stays in bounds: kv_len is clamped to the cache capacity (cache_len,
 * or max_pages * page_size), n_b to [0, min(kv_len[b], max_q)] and to the
 * packed rows that remain, page ids to [0, num_pages); out rows and lse
 * entries that no sequence covers are left untouched.
 * B == 0, total_q == 0 or max_q == 0 is a no-op that returns RA_OK.
 */
int rel_attn_extend(const void* q, const void* k, const void* v, const void* r,
                    const void* P_cols, void* out, float* lse, int dtype,
                    int B, int total_q, int max_q, const int* q_start, const int* kv_len,
                    int cache_len, const int* block_table, int max_pages, int num_pages, int page_size,
                    int Hq, int Hkv, int D, int d_r,
                    float alpha, int rel_extent, int window, int log_scale,
                    void* stream);

/*
 * rel_attn_extend over MXFP8 caches (page "SGLang and Miles Add Day-0
 * Support for Inkling", section "Relative Logits Optimization", paragraph
 * "MXFP8 Support" and Figure 3: the attention kernel reads K and V as MXFP8
 * and takes Q.K^T as an MXFP8 product).  The caches hold E4M3 codes
 * k_codes / v_codes [.., Hkv, D] (uint8, the layout of the dtype caches with
 * one byte per value) and E8M0 scales k_scales / v_scales [.., Hkv, D / 32]
 * (uint8, any alignment), contiguous ([B, cache_len, ...]) or paged
 * ([num_pages, page_size, ...]), as rel_attn_prologue_mx and rel_mx_quantize
 * write them.  q, r, P_cols and out are bf16.  Each new row's query is
 * quantised to MXFP8 as rel_mx_quantize would quantise it, the scores come
 * from the MX-scaled fp8 MFMA, V is dequantised to bf16 (exact) for P.V;
 * the relative bias, masks and softmax are those of rel_attn_extend.
 * Everything else (shapes, q_start / kv_len / block_table, bounds, no-op
 * cases) as rel_attn_extend.
 */
int rel_attn_extend_mx(const void* q, const void* k_codes, const void* k_scales, const void* v_codes,
                       const void* v_scales, const void* r, const void* P_cols, void* out, float* lse,
                       int B, int total_q, int max_q, const int* q_start, const int* kv_len,
                       int cache_len, const int* block_table, int max_pages, int num_pages, int page_size,
                       int Hq, int Hkv, int D, int d_r,
                       float alpha, int rel_extent, int window, int log_scale,
                       void* stream);

/*
 * Attention prologue: the step before the attention kernels on the new
 * tokens' q, k and v projections (page "SGLang and Miles Add Day-0 Support
 * for Inkling", section "ShortConv Optimization", paragraph "KV ShortConv +
 * QK-norm + KV store"), in one kernel:
 *   k' = RMSNorm_k(ShortConv_k(k))  -> k cache
 *   v' = ShortConv_v(v)             -> v cache
 *   q' = RMSNorm_q(q)               -> q_out
 * ShortConv is the filter of section "Short Convolution (ShortConv)":
 * y[t,c] = x[t,c] + sum_{d < conv_width} w[c,d] * x[t-d,c] over the Hkv*D
 * channels of a K (V) row, accumulated in fp32 with the residual added last.
 * RMSNorm is per head over D: x / sqrt(mean(x^2) + eps) * g, with one
 * D-vector g for q and one for k shared by all heads.  r is not touched.
 *   q_in [total_q, Hq, D], k_in and v_in [total_q, Hkv, D]: raw projections,
 *     packed by sequence like extend (rows q_start[b] .. q_start[b+1]-1).
 *   conv_k, conv_v [Hkv*D, conv_width]; q_norm_w, k_norm_w [D]: dtype.
 *   q_out [total_q, Hq, D]: may be q_in itself (in place); no other output
 *     may alias an input.
 *   k_cache, v_cache: the caches of rel_attn_extend / rel_attn_decode_paged
 *     (contiguous [B, cache_len, Hkv, D] when block_table is NULL, else pages
 *     [num_pages, page_size, Hkv, D] with any positive page_size).  New row t
 *     of sequence b goes to position kv_len[b] - n_b + t; rows whose position
 *     falls outside the cache (or on a page id outside [0, num_pages)) are
 *     not written.
 *   state_in, state_out [B, 2, 3, Hkv*D] (dtype) or NULL: the raw K (index
 *     0) and V (index 1) rows of the three positions before the chunk, oldest
 *     first; NULL state_in means zeros (a fresh sequence).  state_out receives
 *     the raw rows of each sequence's last three positions (state_in's rows
 *     carried over for sequences with fewer than three new rows, or none);
 *     state_out must not alias state_in.
 *   q_start [B+1], kv_len [B], block_table [B, max_pages]: int32 device
 *     arrays, 4-byte aligned.  Whatever they hold, every access stays in
 *     bounds (offsets are clamped to [0, total_q]).
 * conv_width in 1 .. 4 (4 in the pages' configurations), eps >= 0.
 * B == 0, or total_q == 0 with state_out NULL, is a no-op that returns RA_OK.
 */
int rel_attn_prologue(const void* q_in, const void* k_in, const void* v_in,
                      const void* conv_k, const void* conv_v,
                      const void* q_norm_w, const void* k_norm_w, float eps,
                      const void* state_in, void* state_out,
                      void* q_out, void* k_cache, void* v_cache, int dtype,
                      int B, int total_q, const int* q_start, const int* kv_len,
                      int cache_len, const int* block_table, int max_pages,
                      int num_pages, int page_size, int Hq, int Hkv, int D,
                      int conv_width, void* stream);

/*
 * Decode plan: a pure function of the shape.  Writes the number of KV splits
 * the decode call will use and the workspace size in bytes the caller must
 * provide.  The split count is the num_splits of the split-KV decode that the
 * vLLM page ("vLLM 宣布 Day-0 支持 TML Inkling 模型", section "vLLM 集成与优化",
 * the paragraph on the sheared-bias FA4 kernel) picks per batch from the
 * batch size, tensor parallelism and KV length: num_splits_req > 0 asks for
 * that many (the plan may use fewer so that every split holds at least one
 * 256-key turn); 0 lets the library choose from B*Hkv, the visible length
 * min(L, window) and the GPU size.  The workspace holds the split partials
 * plus one row of relative logits per (sequence, query head), padded, for
 * the shapes whose bias takes the pre-pass (all zeros when rel_extent == 0).
 * window and rel_extent are inputs because the visible length sets the
 * splits and the extent sets the length of those rows.
 */
int rel_attn_decode_plan(int B, int L, int Hq, int Hkv, int D, int num_splits_req, int window,
                         int rel_extent, int* num_splits_out, size_t* workspace_bytes_out);

/*
 * Decode: one query token per sequence, at position L-1 of its KV cache
 * (the cache already holds that token's own k and v).
 *   q [B, Hq, D]   k, v [B, L, Hkv, D]   r [B, Hq, d_r]   P_cols [E, d_r]
 *   out [B, Hq, D] (dtype)   lse [B, Hq] float32 or NULL
 * num_splits and workspace come from rel_attn_decode_plan with the same shape
 * (workspace: device memory, 256-byte aligned, at least workspace_bytes; its
 * contents on entry are ignored and on return are unspecified).  The KV range
 * is split into num_splits chunks (the split-KV decode of the vLLM page,
 * section "vLLM 集成与优化"); each chunk's partial softmax state is merged by
 * log-sum-exp in a last kernel on the same stream (with one split the split
 * kernel writes out and lse itself).  The workgroups whose chunk holds keys
 * within rel_extent of the query make the bias s * r.P[:, L-1-j] of those
 * keys in LDS; when that region would not fit the LDS budget, a first kernel
 * writes each (sequence, head)'s relative-logit row into the workspace
 * instead and the split kernel adds it by distance.
 */
int rel_attn_decode(const void* q, const void* k, const void* v, const void* r,
                    const void* P_cols, void* out, float* lse, int dtype,
                    int B, int L, int Hq, int Hkv, int D, int d_r,
                    float alpha, int rel_extent, int window, int log_scale,
                    int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * rel_attn_decode without the workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments and results are those of
 * rel_attn_decode (num_splits from rel_attn_decode_plan, or 0); the split
 * partials and bias rows go instead to a fixed scratch array of 16 MiB per
 * device, held by the library from its load to the end of the process.  A
 * shape whose plan needs more (workspace_bytes of rel_attn_decode_plan above
 * 16 MiB) returns RA_ERR_WORKSPACE.  The first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress; nothing is allocated).
 * All calls on one device share its array: calls that overlap on a device
 * (on different streams, or from threads without ordering) race and their
 * results are undefined; calls on one stream are ordered and safe.
 */
int rel_attn_decode_noalloc(const void* q, const void* k, const void* v, const void* r,
                            const void* P_cols, void* out, float* lse, int dtype,
                            int B, int L, int Hq, int Hkv, int D, int d_r,
                            float alpha, int rel_extent, int window, int log_scale,
                            int num_splits, void* stream);

/*
 * Paged decode: one query token per sequence at position kv_len[b]-1 of its
 * paged KV cache, with per-sequence cache lengths (the decode kernels of the
 * serving systems' paged caches).
 *   q [B, Hq, D]   r [B, Hq, d_r]   P_cols [E, d_r]   out [B, Hq, D]   lse [B, Hq] or NULL
 *   k_pages, v_pages [num_pages, page_size, Hkv, D]: key j of sequence b is
 *     slot j % page_size of page block_table[b * max_pages + j / page_size]
 *     (int32 device array [B, max_pages]); page_size a positive multiple of 32.
 *   kv_len [B]: int32 device array of cache lengths, each in [1, max_len].
 * s uses Lseq = kv_len[b] (one scale per sequence, float32 on the device).
 * num_splits and the workspace come from rel_attn_decode_plan with
 * L = max_len; a split past a shorter sequence's keys contributes nothing.
 * The device arrays are not read on the host; whatever they hold, accesses
 * stay in bounds (kv_len clamped to [1, min(max_len, max_pages*page_size)],
 * page ids to [0, num_pages)).
 */
int rel_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const void* r,
                          const void* P_cols, void* out, float* lse, int dtype,
                          int B, int max_len, const int* kv_len, const int* block_table,
                          int max_pages, int num_pages, int page_size,
                          int Hq, int Hkv, int D, int d_r,
                          float alpha, int rel_extent, int window, int log_scale,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP8 K/V (page "SGLang and Miles Add Day-0 Support for Inkling", section
 * "Relative Logits Optimization", paragraph "MXFP8 Support"): K and V stored
 * as OCP MX blocks -- E4M3 codes (one byte per value) with one E8M0 scale
 * byte per 32 values of D (four per 128-wide row), value = E4M3(code) *
 * 2^(scale - 127).  Quantisation of a block: shared exponent =
 * floor(log2(max |x|)) - 8, clamped to [-127, 127] (0 for an all-zero
 * block); each element x * 2^-shared rounded to nearest E4M3, ties to even,
 * magnitudes beyond 448 clamped to 448.
 *
 * rel_mx_quantize: rows of D = 128 values (dtype) -> codes [n_rows, 128]
 * (uint8) and scales [n_rows, 4] (uint8).  x 16-byte aligned; the outputs
 * must not alias x.  n_rows == 0 is a no-op.
 */
int rel_mx_quantize(const void* x, void* codes, void* scales, int dtype,
                    long long n_rows, int D, void* stream);

/*
 * rel_attn_prologue_mx: rel_attn_prologue writing MXFP8 caches: the k and v
 * rows are quantised (as rel_mx_quantize would quantise their fp32 values)
 * into k_codes / v_codes [.., Hkv, D] (uint8, the layout of the dtype caches
 * with one byte per value) and k_scales / v_scales [.., Hkv, D / 32]
 * (uint8), contiguous ([B, cache_len, ...]) or paged ([num_pages,
 * page_size, ...]).  q, k, v, weights, state and q_out are bf16.  The four
 * cache buffers must be distinct.  Everything else as rel_attn_prologue.
 */
int rel_attn_prologue_mx(const void* q_in, const void* k_in, const void* v_in,
                         const void* conv_k, const void* conv_v,
                         const void* q_norm_w, const void* k_norm_w, float eps,
                         const void* state_in, void* state_out, void* q_out,
                         void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                         int B, int total_q, const int* q_start, const int* kv_len,
                         int cache_len, const int* block_table, int max_pages,
                         int num_pages, int page_size, int Hq, int Hkv, int D,
                         int conv_width, void* stream);

/*
 * rel_attn_decode_mx: split-KV decode over MXFP8 caches.  The score product
 * runs on MXFP8 operands: q is quantised like a K row (per (sequence, head)
 * row, blocks of 32 along D) and Q.K^T is taken by the gfx950 MX-scaled
 * fp8 MFMA with fp32 accumulation; V is dequantised to bf16 (exactly) for
 * the bf16 P.V product.  q, r, P_cols, out: bf16; lse float32 or NULL.
 *   Contiguous (block_table == NULL, kv_len == NULL): codes [B, L, Hkv, D],
 *     scales [B, L, Hkv, D / 32]; the query at position L-1, as
 *     rel_attn_decode.
 *   Paged (block_table and kv_len given): codes [num_pages, page_size, Hkv,
 *     D], scales [num_pages, page_size, Hkv, D / 32]; per-sequence lengths
 *     kv_len[b] <= L, as rel_attn_decode_paged (page_size a multiple of 32).
 * Workspace: as rel_attn_decode, sized by rel_attn_decode_plan(B, L, ...).
 */
int rel_attn_decode_mx(const void* q, const void* k_codes, const void* k_scales,
                       const void* v_codes, const void* v_scales, const void* r,
                       const void* P_cols, void* out, float* lse, int B, int L,
                       const int* kv_len, const int* block_table, int max_pages,
                       int num_pages, int page_size, int Hq, int Hkv, int D, int d_r,
                       float alpha, int rel_extent, int window, int log_scale,
                       int num_splits, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Backward plan: a pure function of the shape.  Writes the number of
 * workgroups each kv head's query heads are split over in the dk / dv kernel
 * (head_splits_req > 0 asks for that many and must divide Hq / Hkv; 0 lets
 * the library choose, from the 128-key blocks and B * Hkv, so that the launch
 * fills the GPU) and the workspace size in bytes: delta_i = dout_i . out_i per
 * (sequence, head, row) as float32, plus, when the heads are split, float32
 * partial dk and dv per split.
 */
int rel_attn_backward_plan(int B, int T, int Hq, int Hkv, int D, int head_splits_req,
                           int* head_splits_out, size_t* workspace_bytes_out);

/*
 * Backward of rel_attn_prefill (page "SGLang and Miles Add Day-0 Support for
 * Inkling", section "Customized Efficient Kernels for Train-Inference
 * Consistency", paragraph "Relative attention": gradients through the scores
 * and through r, the relative projection P held fixed).  For the loss
 * sum(dout * out):
 *   dq_i = s alpha sum_j ds_ij k_j        dk_j = s alpha sum_i ds_ij q_i
 *   dv_j = sum_i p_ij dout_i              dr_i = s sum_{d < E} ds_{i,i-d} P[:, d]
 * with p the attention weights, ds_ij = p_ij (dout_i . v_j - dout_i . out_i),
 * and the sums for dk and dv also over the query heads of the kv head.
 *   q, dq, dout, out [B, T, Hq, D]   k, v, dk, dv [B, T, Hkv, D]
 *   r, dr [B, T, Hq, d_r]   P_cols [E, d_r]   lse [B, Hq, T] float32
 * out and lse are what rel_attn_prefill returned for the same inputs and
 * arguments (lse is required).  dtype: RA_BF16 only (RA_F32 returns
 * RA_ERR_UNSUPPORTED); gradients are accumulated in float32 and written in
 * bf16.  rel_extent == 0: r, P_cols and dr may be NULL (a non-NULL dr is left
 * untouched).  head_splits and the workspace come from rel_attn_backward_plan
 * (workspace: device memory, 256-byte aligned, contents ignored on entry and
 * unspecified on return).  Gradient outputs must not alias the inputs, the
 * workspace or each other; they are fully overwritten.  Four kernels on
 * `stream`: delta, dq and dr, dk and dv, and (head_splits > 1) the sum of the
 * partials.  B == 0 or T == 0 is a no-op that returns RA_OK.
 */
int rel_attn_backward(const void* q, const void* k, const void* v, const void* r,
                      const void* P_cols, const void* out, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, void* dr, int dtype,
                      int B, int T, int Hq, int Hkv, int D, int d_r,
                      float alpha, int rel_extent, int window, int log_scale,
                      int head_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense relative logits (eq. for rel_logits in the same section):
 *   out[t, h, d] = s * sum_c r[t, h, c] * P_cols[d, c]   for every d < rel_extent
 *   r [n_tok, H, d_r] (dtype)   P_cols [E, d_r] (dtype)   out [n_tok, H, E] float32
 * s = max(1, ln(seq_len)/ln(4096)) when log_scale, else 1.  No masking.
 */
int rel_logits(const void* r, const void* P_cols, float* out, int dtype,
               long long n_tok, int H, int d_r, int rel_extent, int log_scale,
               long long seq_len, void* stream);

/* The log-scale factor s the library applies for a sequence of seq_len tokens. */
double rel_attn_scale_factor(int log_scale, long long seq_len);

/* Message for the calling thread's last non-zero return ("" if none). */
const char* rel_attn_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int rel_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RELATTN_H */
