// Internal declarations shared by the host API (api.cpp) and the HIP kernel
// sources.  Not part of the public ABI (that is include/relattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace relattn {

constexpr int kHeadDim = 128;
constexpr int kMaxDr = 128;

// Prefill launch description.  Pointers are device pointers; c1 and c2 fold
// the log-scale s, alpha and log2(e) so the kernels work in base 2:
//   c1 = s * alpha * log2(e)   multiplies q.k
//   c2 = s * log2(e)           multiplies r.P
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* r;
  const void* pc;   // P_cols [E, d_r]
  void* out;
  float* lse;       // may be null
  int B, T, Hq, Hkv, d_r, E, W;
  float c1, c2;
  // extend only (see rel_attn_extend); device arrays and their host bounds
  const int* q_start = nullptr;  // [B+1] packed row offsets
  const int* kv_len = nullptr;   // [B] cached tokens per sequence
  const int* btab = nullptr;     // [B, max_pages] page ids, or null (contiguous caches)
  int total_q = 0, max_q = 0;    // packed rows; bound on the new rows of any sequence
  int cap = 0;                   // contiguous caches: rows per sequence
  int max_pages = 0, num_pages = 0, page_size = 0;
  int log_scale = 0;             // s per sequence from kv_len (c1, c2 unused then)
  float alpha = 0.0f;
  // extend over MXFP8 caches (rel_attn_extend_mx): k and v hold E4M3 codes
  // [.., Hkv, D] and these their E8M0 scales [.., Hkv, D / 32]
  const void* k_scale = nullptr;
  const void* v_scale = nullptr;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* r;
  const void* pc;
  void* out;
  float* lse;       // may be null
  float* ws;        // workspace base (float): split partials, then bias rows
  const float* rl;  // bias rows inside the workspace (any valid address when E == 0)
  int B, L, Hq, Hkv, d_r, E, W;
  float c1, c2;
  int n_split;      // splits of the visible key range
  int chunk;        // keys per split (multiple of 32)
  int extra = 0;    // the first n_extra splits hold chunk + extra keys (set by the launcher)
  int n_extra = 0;
  int kv_lo;        // first visible key (L - W for a window, else 0)
  int n_hg;         // groups of 16 query heads per kv head
  int rl_base;      // key j reads bias row entry j - L + rl_base
  int rl_stride;    // floats per bias row
  // bias made in the split kernel (set by the launcher; 0 = pre-pass rows)
  int bias_cols = 0, bias_ld = 0, bias_rows = 0;
  // paged form only (see rel_attn_decode_paged): L is then the bound on kv_len
  const int* kv_len = nullptr;  // [B] cached tokens per sequence
  const int* btab = nullptr;    // [B, max_pages] page ids
  int max_pages = 0, num_pages = 0, page_size = 0;
  int log_scale = 0;            // s per sequence from kv_len
  float alpha = 0.0f;
  // MXFP8 caches only (see rel_attn_decode_mx): k and v then hold E4M3 codes
  // [.., Hkv, D] and these their E8M0 block scales [.., Hkv, D / 32]
  const void* k_scale = nullptr;
  const void* v_scale = nullptr;
};

// Attention prologue (see rel_attn_prologue): device pointers and host bounds.
struct PrologueArgs {
  const void* q_in;
  const void* k_in;
  const void* v_in;
  const void* conv_k;    // [Hkv*D, conv_w]
  const void* conv_v;
  const void* q_norm_w;  // [D]
  const void* k_norm_w;  // [D]
  const void* state_in;  // [B, 2, 3, Hkv*D] or null (zeros)
  void* state_out;       // [B, 2, 3, Hkv*D] or null (not written)
  void* q_out;
  void* k_cache;
  void* v_cache;
  const int* q_start;    // [B+1]
  const int* kv_len;     // [B]
  const int* btab;       // [B, max_pages] or null (contiguous caches of cap rows)
  float eps;
  int B, total_q, Hq, Hkv, conv_w;
  int cap, max_pages, num_pages, page_size;
  // MXFP8 caches (rel_attn_prologue_mx): k_cache / v_cache hold E4M3 codes
  // and these the E8M0 scales [.., Hkv, D / 32]
  void* k_scale = nullptr;
  void* v_scale = nullptr;
};

// out[row * out_stride + oc] = s * r[row] . P_cols[d(oc)] for oc < out_cols,
// with d(oc) = oc, or d(oc) = rev_base - 1 - oc when rev_base > 0; entries
// whose d falls outside [0, E) are written as 0.
struct RelLogitsArgs {
  const void* r;
  const void* pc;
  float* out;
  long long n_rows;  // n_tok * H
  int d_r, E;
  float s;
  int out_cols, out_stride, rev_base;
  // optional per-row shift of the output columns: row r is written from
  // column sh = (4 - Lb % 4) % 4 on, Lb = clamp(shift_len[r / shift_hq], 1,
  // shift_lmax), columns shifted past out_stride dropped (paged decode:
  // aligns each sequence's bias groups)
  const int* shift_len = nullptr;
  int shift_hq = 1, shift_lmax = 1;
};

// Backward launch description (bf16; see rel_attn_backward).  c1 and c2 as
// in PrefillArgs; sa = s * alpha scales dq and dk, s scales dr.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* r;
  const void* pc;    // P_cols [E, d_r]
  const void* out;
  const void* dout;
  const float* lse;  // [B, Hq, T], natural log
  void* dq;
  void* dk;
  void* dv;
  void* dr;          // may be null
  float* delta;      // workspace [B, Hq, T]
  float* part;       // workspace [n_split][2][B, T, Hkv, D] when n_split > 1
  int B, T, Hq, Hkv, d_r, E, W;
  float c1, c2, sa, s;
  int n_split;       // the dk / dv kernel's split of each group's query heads
};

// Decode planning shared by rel_attn_decode_plan and rel_attn_decode.
struct DecodePlan {
  int n_split;
  int chunk;
  int kv_lo;
  int n_hg;
  int rl_base;
  int rl_stride;
  size_t ws_partial_bytes;  // split partials (o, m, l)
  size_t ws_bytes;          // total, bias rows included
};
DecodePlan plan_decode(int B, int L, int Hq, int Hkv, int num_splits_req, int window, int rel_extent);

// Launchers: return hipSuccess or the launch error.  dtype: 1 = bf16, 2 = fp32.
hipError_t launch_prefill(int dtype, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prologue(int dtype, const PrologueArgs& a, hipStream_t stream);
// bf16 inputs, MXFP8 caches
hipError_t launch_prologue_mx(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_extend(int dtype, const PrefillArgs& a, hipStream_t stream);
// bf16 q / r / P / out, MXFP8 caches
hipError_t launch_extend_mx(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_paged(int dtype, const DecodeArgs& a, hipStream_t stream);
// MXFP8 K/V caches, bf16 q / r / P / out; paged when a.btab is set
hipError_t launch_decode_mx(const DecodeArgs& a, hipStream_t stream);
// rows of D = 128 values (dtype) -> E4M3 codes [n_rows, 128] and E8M0 scales [n_rows, 4]
hipError_t launch_mx_quantize(int dtype, const void* x, void* codes, void* scales, long long n_rows, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_rel_logits(int dtype, const RelLogitsArgs& a, hipStream_t stream);

}  // namespace relattn
