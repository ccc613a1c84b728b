// Host side of the C ABI declared in include/relattn.h: argument checks (all
// before any HIP call), the log-scale factor, decode planning, launches and
// per-thread error messages.  No device memory is allocated here and no
// device data is read on the host.
#include "relattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "relattn_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return RA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* name, bool required) {
  if (p == nullptr) {
    if (required) return fail(RA_ERR_INVALID_ARG, "%s is NULL", name);
    return RA_OK;
  }
  if (!aligned16(p)) return fail(RA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return RA_OK;
}

double scale_of(int log_scale, long long len) {
  if (!log_scale || len <= 1) return 1.0;
  const double s = std::log((double)len) / std::log(4096.0);
  return s > 1.0 ? s : 1.0;
}

// Checks common to prefill and decode.
int check_common(int dtype, int B, int Tl, int Hq, int Hkv, int D, int d_r, float alpha, int rel_extent,
                 int window, int log_scale, const char* len_name) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_BF16 or RA_F32", dtype);
  if (B < 0) return fail(RA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (Tl < 0) return fail(RA_ERR_INVALID_ARG, "%s = %d < 0", len_name, Tl);
  if (Hq <= 0 || Hkv <= 0) return fail(RA_ERR_INVALID_ARG, "Hq = %d and Hkv = %d must be positive", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(RA_ERR_INVALID_ARG, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  if (rel_extent < 0) return fail(RA_ERR_INVALID_ARG, "rel_extent = %d < 0", rel_extent);
  if (window < 0) return fail(RA_ERR_INVALID_ARG, "window = %d < 0", window);
  if (log_scale != 0 && log_scale != 1) return fail(RA_ERR_INVALID_ARG, "log_scale = %d is not 0 or 1", log_scale);
  if (!std::isfinite(alpha)) return fail(RA_ERR_INVALID_ARG, "alpha is not finite");
  if (D != relattn::kHeadDim) return fail(RA_ERR_UNSUPPORTED, "head dim D = %d: only 128 is supported", D);
  if (rel_extent > 0) {
    if (d_r <= 0 || d_r % 16 != 0 || d_r > relattn::kMaxDr)
      return fail(RA_ERR_UNSUPPORTED, "d_r = %d: supported values are multiples of 16 in [16, 128]", d_r);
  }
  return RA_OK;
}

// ---- decode: the checks (host only, before any HIP call) and the launch,
// shared by rel_attn_decode and rel_attn_decode_noalloc
int decode_check(const void* q, const void* k, const void* v, const void* r, const void* P_cols, void* out,
                 float* lse, int dtype, int B, int L, int Hq, int Hkv, int D, int d_r, float alpha, int rel_extent,
                 int window, int log_scale, int num_splits, relattn::DecodePlan* pl) {
  int rc = check_common(dtype, B, L, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "L");
  if (rc) return rc;
  if (L == 0) return fail(RA_ERR_INVALID_ARG, "L = 0: the cache must hold at least the query's own token");
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k, "k", true)) || (rc = check_ptr(v, "v", true)) ||
      (rc = check_ptr(out, "out", true)) || (rc = check_ptr(lse, "lse", false)) ||
      (rc = check_ptr(r, "r", rel_extent > 0)) || (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)))
    return rc;
  if (out == q || out == k || out == v || out == r) return fail(RA_ERR_INVALID_ARG, "out aliases an input");
  if (num_splits < 0) return fail(RA_ERR_INVALID_ARG, "num_splits = %d < 0", num_splits);
  if ((long long)B * L > 0x7fffffffLL)
    return fail(RA_ERR_UNSUPPORTED, "B * L = %lld too large", (long long)B * L);
  *pl = relattn::plan_decode(B, L, Hq, Hkv, num_splits, window, rel_extent);
  return RA_OK;
}

int decode_launch(const void* q, const void* k, const void* v, const void* r, const void* P_cols, void* out,
                  float* lse, int dtype, int B, int L, int Hq, int Hkv, int d_r, float alpha, int rel_extent,
                  int window, int log_scale, const relattn::DecodePlan& pl, void* workspace, void* stream) {
  const double s = scale_of(log_scale, L);
  relattn::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.r = r; a.pc = P_cols; a.out = out; a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 16; a.E = rel_extent; a.W = window;
  a.c1 = (float)(s * (double)alpha * 1.4426950408889634);
  a.c2 = (float)(s * 1.4426950408889634);
  a.n_split = pl.n_split;
  a.chunk = pl.chunk;
  a.kv_lo = pl.kv_lo;
  a.n_hg = pl.n_hg;
  a.rl_base = pl.rl_base;
  a.rl_stride = pl.rl_stride;
  a.rl = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.ws_partial_bytes);
  hipError_t e = relattn::launch_decode(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---- the fixed scratch of rel_attn_decode_noalloc: one array per device,
// held from the library's load to the end of the process.  In host code the
// array's name stands for the device copy only through hipGetSymbolAddress,
// which is called once per device (with that device current) and cached.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_stream(void* stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return fail(RA_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(RA_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr)
      return fail(RA_ERR_HIP, "hipGetSymbolAddress of the decode scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

// ---- extend with caches in the input dtype, or in MXFP8 (mx: E4M3 codes in
// k / v and their E8M0 scales; bf16 q, r, P and out)
int extend_impl(const void* q, const void* k, const void* k_scales, const void* v, const void* v_scales, bool mx,
                const void* r, const void* P_cols, void* out, float* lse, int dtype, int B, int total_q, int max_q,
                const int* q_start, const int* kv_len, int cache_len, const int* block_table, int max_pages,
                int num_pages, int page_size, int Hq, int Hkv, int D, int d_r, float alpha, int rel_extent,
                int window, int log_scale, void* stream) {
  int rc = check_common(dtype, B, total_q, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "total_q");
  if (rc) return rc;
  if (max_q < 0) return fail(RA_ERR_INVALID_ARG, "max_q = %d < 0", max_q);
  if (B == 0 || total_q == 0 || max_q == 0) return ok();
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k, "k", true)) || (rc = check_ptr(v, "v", true)) ||
      (rc = check_ptr(out, "out", true)) || (rc = check_ptr(lse, "lse", false)) ||
      (rc = check_ptr(r, "r", rel_extent > 0)) || (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)))
    return rc;
  if (mx && (k_scales == nullptr || v_scales == nullptr))
    return fail(RA_ERR_INVALID_ARG, "k_scales and v_scales must not be NULL");
  if (q_start == nullptr || kv_len == nullptr) return fail(RA_ERR_INVALID_ARG, "q_start and kv_len must not be NULL");
  if ((reinterpret_cast<uintptr_t>(q_start) | reinterpret_cast<uintptr_t>(kv_len) |
       reinterpret_cast<uintptr_t>(block_table)) & 3u)
    return fail(RA_ERR_INVALID_ARG, "q_start, kv_len and block_table must be 4-byte aligned");
  {
    const void* ins[7] = {q, k, v, r, P_cols, k_scales, v_scales};
    for (const void* i : ins)
      if (i != nullptr && (i == out || i == lse)) return fail(RA_ERR_INVALID_ARG, "out or lse aliases an input");
  }
  if (block_table == nullptr) {
    if (cache_len <= 0) return fail(RA_ERR_INVALID_ARG, "cache_len = %d: contiguous caches need cache_len >= 1", cache_len);
  } else {
    if (page_size <= 0 || page_size % 32 != 0)
      return fail(RA_ERR_UNSUPPORTED, "page_size = %d: supported values are positive multiples of 32", page_size);
    if (max_pages <= 0 || num_pages <= 0)
      return fail(RA_ERR_INVALID_ARG, "max_pages = %d and num_pages = %d must be positive", max_pages, num_pages);
    if ((long long)max_pages * page_size > 0x7fffffffLL)
      return fail(RA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  }
  if ((long long)total_q * Hq > 0x7fffffffLL / relattn::kHeadDim)
    return fail(RA_ERR_UNSUPPORTED, "total_q * Hq = %lld too large for one launch", (long long)total_q * Hq);

  relattn::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.r = r; a.pc = P_cols; a.out = out; a.lse = lse;
  a.B = B; a.T = 0; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 16; a.E = rel_extent; a.W = window;
  a.c1 = (float)((double)alpha * 1.4426950408889634);
  a.c2 = (float)1.4426950408889634;
  a.q_start = q_start; a.kv_len = kv_len; a.btab = block_table;
  a.total_q = total_q; a.max_q = max_q; a.cap = block_table == nullptr ? cache_len : 0;
  a.max_pages = max_pages; a.num_pages = num_pages; a.page_size = page_size;
  a.log_scale = log_scale; a.alpha = alpha;
  a.k_scale = k_scales; a.v_scale = v_scales;
  hipError_t e = mx ? relattn::launch_extend_mx(a, static_cast<hipStream_t>(stream))
                    : relattn::launch_extend(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "extend launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* rel_attn_last_error(void) { return g_err; }

int rel_attn_version(void) { return 100; }  // 0.1.0

double rel_attn_scale_factor(int log_scale, long long seq_len) { return scale_of(log_scale, seq_len); }

int rel_attn_prefill(const void* q, const void* k, const void* v, const void* r, const void* P_cols, void* out,
                     float* lse, int dtype, int B, int T, int Hq, int Hkv, int D, int d_r, float alpha,
                     int rel_extent, int window, int log_scale, void* stream) {
  int rc = check_common(dtype, B, T, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "T");
  if (rc) return rc;
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k, "k", true)) || (rc = check_ptr(v, "v", true)) ||
      (rc = check_ptr(out, "out", true)) || (rc = check_ptr(lse, "lse", false)) ||
      (rc = check_ptr(r, "r", rel_extent > 0)) || (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)))
    return rc;
  if (out == q || out == k || out == v || out == r) return fail(RA_ERR_INVALID_ARG, "out aliases an input");
  if ((long long)T * Hq > 0x7fffffffLL / relattn::kHeadDim)
    return fail(RA_ERR_UNSUPPORTED, "T * Hq = %lld too large for one launch", (long long)T * Hq);
  if (B == 0 || T == 0) return ok();

  const double s = scale_of(log_scale, T);
  relattn::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.r = r; a.pc = P_cols; a.out = out; a.lse = lse;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 16; a.E = rel_extent; a.W = window;
  a.c1 = (float)(s * (double)alpha * 1.4426950408889634);
  a.c2 = (float)(s * 1.4426950408889634);
  hipError_t e = relattn::launch_prefill(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rel_attn_extend(const void* q, const void* k, const void* v, const void* r, const void* P_cols, void* out,
                    float* lse, int dtype, int B, int total_q, int max_q, const int* q_start, const int* kv_len,
                    int cache_len, const int* block_table, int max_pages, int num_pages, int page_size, int Hq,
                    int Hkv, int D, int d_r, float alpha, int rel_extent, int window, int log_scale, void* stream) {
  return extend_impl(q, k, nullptr, v, nullptr, false, r, P_cols, out, lse, dtype, B, total_q, max_q, q_start, kv_len,
                     cache_len, block_table, max_pages, num_pages, page_size, Hq, Hkv, D, d_r, alpha, rel_extent,
                     window, log_scale, stream);
}

int rel_attn_extend_mx(const void* q, const void* k_codes, const void* k_scales, const void* v_codes,
                       const void* v_scales, const void* r, const void* P_cols, void* out, float* lse, int B,
                       int total_q, int max_q, const int* q_start, const int* kv_len, int cache_len,
                       const int* block_table, int max_pages, int num_pages, int page_size, int Hq, int Hkv, int D,
                       int d_r, float alpha, int rel_extent, int window, int log_scale, void* stream) {
  return extend_impl(q, k_codes, k_scales, v_codes, v_scales, true, r, P_cols, out, lse, RA_BF16, B, total_q, max_q,
                     q_start, kv_len, cache_len, block_table, max_pages, num_pages, page_size, Hq, Hkv, D, d_r, alpha,
                     rel_extent, window, log_scale, stream);
}

}  // extern "C"

namespace {

// The prologue with caches in the input dtype (k_scale == v_scale == NULL) or
// in MXFP8 (E4M3 codes in k_cache / v_cache and their E8M0 scales).
int prologue_impl(const void* q_in, const void* k_in, const void* v_in, const void* conv_k, const void* conv_v,
                  const void* q_norm_w, const void* k_norm_w, float eps, const void* state_in, void* state_out,
                  void* q_out, void* k_cache, void* v_cache, bool mx, void* k_scale, void* v_scale, int dtype,
                  int B, int total_q, const int* q_start, const int* kv_len, int cache_len, const int* block_table,
                  int max_pages, int num_pages, int page_size, int Hq, int Hkv, int D, int conv_width,
                  void* stream) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_BF16 or RA_F32", dtype);
  if (B < 0) return fail(RA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (total_q < 0) return fail(RA_ERR_INVALID_ARG, "total_q = %d < 0", total_q);
  if (Hq <= 0 || Hkv <= 0) return fail(RA_ERR_INVALID_ARG, "Hq = %d and Hkv = %d must be positive", Hq, Hkv);
  if (D != relattn::kHeadDim) return fail(RA_ERR_UNSUPPORTED, "head dim D = %d: only 128 is supported", D);
  if (conv_width < 1 || conv_width > 4)
    return fail(RA_ERR_UNSUPPORTED, "conv_width = %d: supported widths are 1 .. 4", conv_width);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(RA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  // With no new row the call only carries the states of the B sequences over.
  if (B == 0 || (total_q == 0 && state_out == nullptr)) return ok();
  const bool rows = total_q > 0;
  int rc;
  if ((rc = check_ptr(q_in, "q_in", rows)) || (rc = check_ptr(k_in, "k_in", rows)) ||
      (rc = check_ptr(v_in, "v_in", rows)) || (rc = check_ptr(q_out, "q_out", rows)) ||
      (rc = check_ptr(k_cache, "k_cache", rows)) || (rc = check_ptr(v_cache, "v_cache", rows)) ||
      (rc = check_ptr(q_norm_w, "q_norm_w", rows)) || (rc = check_ptr(k_norm_w, "k_norm_w", rows)) ||
      (rc = check_ptr(state_in, "state_in", false)) || (rc = check_ptr(state_out, "state_out", false)))
    return rc;
  if (rows && (conv_k == nullptr || conv_v == nullptr))
    return fail(RA_ERR_INVALID_ARG, "conv_k and conv_v must not be NULL");
  const size_t esz = dtype == RA_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(conv_k) | reinterpret_cast<uintptr_t>(conv_v)) & (esz - 1))
    return fail(RA_ERR_INVALID_ARG, "conv_k and conv_v must be aligned to the element size");
  if (q_start == nullptr || kv_len == nullptr) return fail(RA_ERR_INVALID_ARG, "q_start and kv_len must not be NULL");
  if ((reinterpret_cast<uintptr_t>(q_start) | reinterpret_cast<uintptr_t>(kv_len) |
       reinterpret_cast<uintptr_t>(block_table)) & 3u)
    return fail(RA_ERR_INVALID_ARG, "q_start, kv_len and block_table must be 4-byte aligned");
  if (state_out != nullptr && state_out == state_in)
    return fail(RA_ERR_INVALID_ARG, "state_out aliases state_in (the new state would overwrite rows still to be read)");
  if (rows && k_cache == v_cache) return fail(RA_ERR_INVALID_ARG, "k_cache and v_cache are the same buffer");
  const void* outs[3] = {k_cache, v_cache, state_out};
  const void* ins[5] = {q_in, k_in, v_in, state_in, q_norm_w};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o != nullptr && o == i) return fail(RA_ERR_INVALID_ARG, "an output buffer aliases an input");
  if (rows && (q_out == k_in || q_out == v_in)) return fail(RA_ERR_INVALID_ARG, "q_out aliases k_in or v_in");
  if (mx && rows) {
    if (k_scale == nullptr || v_scale == nullptr) return fail(RA_ERR_INVALID_ARG, "k_scales and v_scales must not be NULL");
    const void* mouts[4] = {k_cache, v_cache, k_scale, v_scale};
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (mouts[i] == mouts[j]) return fail(RA_ERR_INVALID_ARG, "the MXFP8 code and scale buffers overlap");
    for (const void* i : ins)
      if (i == k_scale || i == v_scale) return fail(RA_ERR_INVALID_ARG, "an output buffer aliases an input");
  }
  if (!rows) {
    // only the state copies run; the cache geometry is not used
  } else if (block_table == nullptr) {
    if (cache_len <= 0) return fail(RA_ERR_INVALID_ARG, "cache_len = %d: contiguous caches need cache_len >= 1", cache_len);
  } else {
    if (page_size <= 0) return fail(RA_ERR_INVALID_ARG, "page_size = %d must be positive", page_size);
    if (max_pages <= 0 || num_pages <= 0)
      return fail(RA_ERR_INVALID_ARG, "max_pages = %d and num_pages = %d must be positive", max_pages, num_pages);
    if ((long long)max_pages * page_size > 0x7fffffffLL)
      return fail(RA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  }
  if ((long long)total_q * (Hq + 2LL * Hkv) / 16 + (long long)B * 2 * Hkv > 0x7fffffffLL - 16)
    return fail(RA_ERR_UNSUPPORTED, "total_q = %d too large for one launch", total_q);

  relattn::PrologueArgs a;
  a.q_in = q_in; a.k_in = k_in; a.v_in = v_in; a.conv_k = conv_k; a.conv_v = conv_v;
  a.q_norm_w = q_norm_w; a.k_norm_w = k_norm_w; a.state_in = state_in; a.state_out = state_out;
  a.q_out = q_out; a.k_cache = k_cache; a.v_cache = v_cache;
  a.q_start = q_start; a.kv_len = kv_len; a.btab = block_table;
  a.eps = eps; a.B = B; a.total_q = total_q; a.Hq = Hq; a.Hkv = Hkv; a.conv_w = conv_width;
  a.cap = block_table == nullptr ? cache_len : 0;
  a.max_pages = block_table == nullptr ? 0 : max_pages;
  a.num_pages = block_table == nullptr ? 0 : num_pages;
  a.page_size = block_table == nullptr ? 1 : page_size;
  a.k_scale = k_scale; a.v_scale = v_scale;
  hipError_t e = mx ? relattn::launch_prologue_mx(a, static_cast<hipStream_t>(stream))
                    : relattn::launch_prologue(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int rel_attn_prologue(const void* q_in, const void* k_in, const void* v_in, const void* conv_k, const void* conv_v,
                      const void* q_norm_w, const void* k_norm_w, float eps, const void* state_in, void* state_out,
                      void* q_out, void* k_cache, void* v_cache, int dtype, int B, int total_q, const int* q_start,
                      const int* kv_len, int cache_len, const int* block_table, int max_pages, int num_pages,
                      int page_size, int Hq, int Hkv, int D, int conv_width, void* stream) {
  return prologue_impl(q_in, k_in, v_in, conv_k, conv_v, q_norm_w, k_norm_w, eps, state_in, state_out, q_out,
                       k_cache, v_cache, false, nullptr, nullptr, dtype, B, total_q, q_start, kv_len, cache_len,
                       block_table, max_pages, num_pages, page_size, Hq, Hkv, D, conv_width, stream);
}

int rel_attn_prologue_mx(const void* q_in, const void* k_in, const void* v_in, const void* conv_k,
                         const void* conv_v, const void* q_norm_w, const void* k_norm_w, float eps,
                         const void* state_in, void* state_out, void* q_out, void* k_codes, void* k_scales,
                         void* v_codes, void* v_scales, int B, int total_q, const int* q_start, const int* kv_len,
                         int cache_len, const int* block_table, int max_pages, int num_pages, int page_size, int Hq,
                         int Hkv, int D, int conv_width, void* stream) {
  return prologue_impl(q_in, k_in, v_in, conv_k, conv_v, q_norm_w, k_norm_w, eps, state_in, state_out, q_out,
                       k_codes, v_codes, true, k_scales, v_scales, RA_BF16, B, total_q, q_start, kv_len, cache_len,
                       block_table, max_pages, num_pages, page_size, Hq, Hkv, D, conv_width, stream);
}

namespace {
// Backward planning: the dk / dv kernel runs one workgroup per 128-key block,
// kv head and split of the group's query heads; the split doubles until the
// launch has a workgroup for every compute unit (or the group is exhausted).
constexpr size_t kBwdAlign = 256;
int bwd_splits(int B, int T, int Hq, int Hkv, int req) {
  const int G = Hq / Hkv;
  if (req > 0) return req;
  const long long n_kb = (T + 127) / 128;
  int n = 1;
  while (n_kb * B * Hkv * n < 256 && G % (n * 2) == 0) n *= 2;
  return n;
}
size_t bwd_delta_bytes(int B, int T, int Hq) {
  return ((size_t)B * Hq * T * sizeof(float) + kBwdAlign - 1) / kBwdAlign * kBwdAlign;
}
size_t bwd_ws_bytes(int B, int T, int Hq, int Hkv, int n_split) {
  const size_t part = n_split > 1 ? (size_t)n_split * 2 * B * T * Hkv * relattn::kHeadDim * sizeof(float) : 0;
  return bwd_delta_bytes(B, T, Hq) + part;
}
}  // namespace

int rel_attn_backward_plan(int B, int T, int Hq, int Hkv, int D, int head_splits_req, int* head_splits_out,
                           size_t* workspace_bytes_out) {
  if (head_splits_out == nullptr || workspace_bytes_out == nullptr)
    return fail(RA_ERR_INVALID_ARG, "head_splits_out and workspace_bytes_out must not be NULL");
  if (B < 0 || T < 0) return fail(RA_ERR_INVALID_ARG, "B = %d, T = %d must not be negative", B, T);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(RA_ERR_INVALID_ARG, "Hq = %d, Hkv = %d: need positive Hq multiple of Hkv", Hq, Hkv);
  if (D != relattn::kHeadDim) return fail(RA_ERR_UNSUPPORTED, "head dim D = %d: only 128 is supported", D);
  if (head_splits_req < 0 || (head_splits_req > 0 && (Hq / Hkv) % head_splits_req != 0))
    return fail(RA_ERR_INVALID_ARG, "head_splits = %d must be 0 or divide Hq / Hkv = %d", head_splits_req, Hq / Hkv);
  const int n = bwd_splits(B, T, Hq, Hkv, head_splits_req);
  *head_splits_out = n;
  *workspace_bytes_out = bwd_ws_bytes(B, T, Hq, Hkv, n);
  return ok();
}

int rel_attn_backward(const void* q, const void* k, const void* v, const void* r, const void* P_cols,
                      const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv, void* dr,
                      int dtype, int B, int T, int Hq, int Hkv, int D, int d_r, float alpha, int rel_extent,
                      int window, int log_scale, int head_splits, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = check_common(dtype, B, T, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "T");
  if (rc) return rc;
  if (dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "backward: only RA_BF16 is supported");
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k, "k", true)) || (rc = check_ptr(v, "v", true)) ||
      (rc = check_ptr(out, "out", true)) || (rc = check_ptr(dout, "dout", true)) ||
      (rc = check_ptr(lse, "lse", true)) || (rc = check_ptr(dq, "dq", true)) || (rc = check_ptr(dk, "dk", true)) ||
      (rc = check_ptr(dv, "dv", true)) || (rc = check_ptr(r, "r", rel_extent > 0)) ||
      (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)) || (rc = check_ptr(dr, "dr", rel_extent > 0)))
    return rc;
  const void* ins[] = {q, k, v, r, P_cols, out, dout, lse, workspace};
  const void* outs[] = {dq, dk, dv, dr};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o != nullptr && o == i) return fail(RA_ERR_INVALID_ARG, "a gradient output aliases an input or the workspace");
  if (dq == dk || dq == dv || dk == dv || (dr != nullptr && (dr == dq || dr == dk || dr == dv)))
    return fail(RA_ERR_INVALID_ARG, "gradient outputs alias each other");
  if ((long long)T * Hq > 0x7fffffffLL / relattn::kHeadDim)
    return fail(RA_ERR_UNSUPPORTED, "T * Hq = %lld too large for one launch", (long long)T * Hq);
  if (head_splits <= 0 || (Hq / Hkv) % head_splits != 0)
    return fail(RA_ERR_INVALID_ARG, "head_splits = %d must divide Hq / Hkv = %d (see rel_attn_backward_plan)",
                head_splits, Hq / Hkv);
  if (B == 0 || T == 0) return ok();
  const size_t need = bwd_ws_bytes(B, T, Hq, Hkv, head_splits);
  if (workspace == nullptr) return fail(RA_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kBwdAlign - 1)) != 0)
    return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);

  const double s = scale_of(log_scale, T);
  relattn::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.r = r; a.pc = P_cols; a.out = out; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dr = rel_extent > 0 ? dr : nullptr;
  a.delta = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(B, T, Hq));
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 0; a.E = rel_extent; a.W = window;
  a.c1 = (float)(s * (double)alpha * 1.4426950408889634);
  a.c2 = (float)(s * 1.4426950408889634);
  a.sa = (float)(s * (double)alpha);
  a.s = (float)s;
  a.n_split = head_splits;
  hipError_t e = relattn::launch_backward(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rel_attn_decode_plan(int B, int L, int Hq, int Hkv, int D, int num_splits_req, int window, int rel_extent,
                         int* num_splits_out, size_t* workspace_bytes_out) {
  if (num_splits_out == nullptr || workspace_bytes_out == nullptr)
    return fail(RA_ERR_INVALID_ARG, "num_splits_out and workspace_bytes_out must not be NULL");
  if (B < 0) return fail(RA_ERR_INVALID_ARG, "B = %d < 0", B);
  if (L <= 0) return fail(RA_ERR_INVALID_ARG, "L = %d: the cache must hold at least the query's own token", L);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(RA_ERR_INVALID_ARG, "Hq = %d, Hkv = %d: need positive Hq multiple of Hkv", Hq, Hkv);
  if (window < 0) return fail(RA_ERR_INVALID_ARG, "window = %d < 0", window);
  if (num_splits_req < 0) return fail(RA_ERR_INVALID_ARG, "num_splits = %d < 0", num_splits_req);
  if (rel_extent < 0) return fail(RA_ERR_INVALID_ARG, "rel_extent = %d < 0", rel_extent);
  if (D != relattn::kHeadDim) return fail(RA_ERR_UNSUPPORTED, "head dim D = %d: only 128 is supported", D);
  relattn::DecodePlan pl = relattn::plan_decode(B, L, Hq, Hkv, num_splits_req, window, rel_extent);
  *num_splits_out = pl.n_split;
  *workspace_bytes_out = pl.ws_bytes;
  return ok();
}

int rel_attn_decode(const void* q, const void* k, const void* v, const void* r, const void* P_cols, void* out,
                    float* lse, int dtype, int B, int L, int Hq, int Hkv, int D, int d_r, float alpha,
                    int rel_extent, int window, int log_scale, int num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  relattn::DecodePlan pl;
  int rc = decode_check(q, k, v, r, P_cols, out, lse, dtype, B, L, Hq, Hkv, D, d_r, alpha, rel_extent, window,
                        log_scale, num_splits, &pl);
  if (rc) return rc;
  if (B == 0) return ok();
  if (workspace == nullptr) return fail(RA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.ws_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < pl.ws_bytes)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu the plan needs", workspace_bytes,
                pl.ws_bytes);
  return decode_launch(q, k, v, r, P_cols, out, lse, dtype, B, L, Hq, Hkv, d_r, alpha, rel_extent, window, log_scale,
                       pl, workspace, stream);
}

int rel_attn_decode_noalloc(const void* q, const void* k, const void* v, const void* r, const void* P_cols,
                            void* out, float* lse, int dtype, int B, int L, int Hq, int Hkv, int D, int d_r,
                            float alpha, int rel_extent, int window, int log_scale, int num_splits, void* stream) {
  relattn::DecodePlan pl;
  int rc = decode_check(q, k, v, r, P_cols, out, lse, dtype, B, L, Hq, Hkv, D, d_r, alpha, rel_extent, window,
                        log_scale, num_splits, &pl);
  if (rc) return rc;
  if (B == 0) return ok();
  if (pl.ws_bytes > kNoAllocScratchBytes)
    return fail(RA_ERR_WORKSPACE, "this decode needs %zu bytes of scratch; the fixed scratch holds %zu (use "
                "rel_attn_decode with a workspace)", pl.ws_bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_stream(stream, &ws))) return rc;
  return decode_launch(q, k, v, r, P_cols, out, lse, dtype, B, L, Hq, Hkv, d_r, alpha, rel_extent, window, log_scale,
                       pl, ws, stream);
}

int rel_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const void* r,
                          const void* P_cols, void* out, float* lse, int dtype, int B, int max_len,
                          const int* kv_len, const int* block_table, int max_pages, int num_pages, int page_size,
                          int Hq, int Hkv, int D, int d_r, float alpha, int rel_extent, int window, int log_scale,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(dtype, B, max_len, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "max_len");
  if (rc) return rc;
  if (max_len == 0) return fail(RA_ERR_INVALID_ARG, "max_len = 0: a cache holds at least the query's own token");
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k_pages, "k_pages", true)) ||
      (rc = check_ptr(v_pages, "v_pages", true)) || (rc = check_ptr(out, "out", true)) ||
      (rc = check_ptr(lse, "lse", false)) || (rc = check_ptr(r, "r", rel_extent > 0)) ||
      (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)))
    return rc;
  if (kv_len == nullptr || block_table == nullptr)
    return fail(RA_ERR_INVALID_ARG, "kv_len and block_table must not be NULL");
  if ((reinterpret_cast<uintptr_t>(kv_len) | reinterpret_cast<uintptr_t>(block_table)) & 3u)
    return fail(RA_ERR_INVALID_ARG, "kv_len and block_table must be 4-byte aligned");
  if (out == q || out == k_pages || out == v_pages || out == r) return fail(RA_ERR_INVALID_ARG, "out aliases an input");
  if (page_size <= 0 || page_size % 32 != 0)
    return fail(RA_ERR_UNSUPPORTED, "page_size = %d: supported values are positive multiples of 32", page_size);
  if (max_pages <= 0 || num_pages <= 0)
    return fail(RA_ERR_INVALID_ARG, "max_pages = %d and num_pages = %d must be positive", max_pages, num_pages);
  if ((long long)max_pages * page_size > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  if (num_splits < 0) return fail(RA_ERR_INVALID_ARG, "num_splits = %d < 0", num_splits);
  relattn::DecodePlan pl = relattn::plan_decode(B, max_len, Hq, Hkv, num_splits, window, rel_extent);
  if (B == 0) return ok();
  if (workspace == nullptr) return fail(RA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.ws_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < pl.ws_bytes)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu the plan needs", workspace_bytes,
                pl.ws_bytes);

  relattn::DecodeArgs a;
  a.q = q; a.k = k_pages; a.v = v_pages; a.r = r; a.pc = P_cols; a.out = out; a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.B = B; a.L = max_len; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 16; a.E = rel_extent; a.W = window;
  a.c1 = (float)((double)alpha * 1.4426950408889634);
  a.c2 = (float)1.4426950408889634;
  a.n_split = pl.n_split;
  a.chunk = pl.chunk;
  a.kv_lo = pl.kv_lo;
  a.n_hg = pl.n_hg;
  a.rl_base = pl.rl_base;
  a.rl_stride = pl.rl_stride;
  a.rl = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.ws_partial_bytes);
  a.kv_len = kv_len; a.btab = block_table;
  a.max_pages = max_pages; a.num_pages = num_pages; a.page_size = page_size;
  a.log_scale = log_scale; a.alpha = alpha;
  hipError_t e = relattn::launch_decode_paged(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rel_attn_decode_mx(const void* q, const void* k_codes, const void* k_scales, const void* v_codes,
                       const void* v_scales, const void* r, const void* P_cols, void* out, float* lse, int B, int L,
                       const int* kv_len, const int* block_table, int max_pages, int num_pages, int page_size, int Hq,
                       int Hkv, int D, int d_r, float alpha, int rel_extent, int window, int log_scale,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(RA_BF16, B, L, Hq, Hkv, D, d_r, alpha, rel_extent, window, log_scale, "L");
  if (rc) return rc;
  if (L == 0) return fail(RA_ERR_INVALID_ARG, "L = 0: a cache holds at least the query's own token");
  if ((rc = check_ptr(q, "q", true)) || (rc = check_ptr(k_codes, "k_codes", true)) ||
      (rc = check_ptr(v_codes, "v_codes", true)) || (rc = check_ptr(out, "out", true)) ||
      (rc = check_ptr(lse, "lse", false)) || (rc = check_ptr(r, "r", rel_extent > 0)) ||
      (rc = check_ptr(P_cols, "P_cols", rel_extent > 0)))
    return rc;
  if (k_scales == nullptr || v_scales == nullptr) return fail(RA_ERR_INVALID_ARG, "k_scales and v_scales must not be NULL");
  const bool paged = block_table != nullptr;
  if (paged) {
    if (kv_len == nullptr) return fail(RA_ERR_INVALID_ARG, "a paged cache needs kv_len");
    if ((reinterpret_cast<uintptr_t>(kv_len) | reinterpret_cast<uintptr_t>(block_table)) & 3u)
      return fail(RA_ERR_INVALID_ARG, "kv_len and block_table must be 4-byte aligned");
    if (page_size <= 0 || page_size % 32 != 0)
      return fail(RA_ERR_UNSUPPORTED, "page_size = %d: supported values are positive multiples of 32", page_size);
    if (max_pages <= 0 || num_pages <= 0)
      return fail(RA_ERR_INVALID_ARG, "max_pages = %d and num_pages = %d must be positive", max_pages, num_pages);
    if ((long long)max_pages * page_size > 0x7fffffffLL)
      return fail(RA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  } else if (kv_len != nullptr) {
    return fail(RA_ERR_INVALID_ARG, "kv_len is for paged caches; a contiguous cache holds L keys per sequence");
  }
  const void* ins[7] = {q, k_codes, k_scales, v_codes, v_scales, r, P_cols};
  for (const void* i : ins)
    if (i != nullptr && (i == out || i == lse)) return fail(RA_ERR_INVALID_ARG, "out or lse aliases an input");
  if (num_splits < 0) return fail(RA_ERR_INVALID_ARG, "num_splits = %d < 0", num_splits);
  relattn::DecodePlan pl = relattn::plan_decode(B, L, Hq, Hkv, num_splits, window, rel_extent);
  if (B == 0) return ok();
  if (workspace == nullptr) return fail(RA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", pl.ws_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(RA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < pl.ws_bytes)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu the plan needs", workspace_bytes,
                pl.ws_bytes);
  if (!paged && (long long)B * L > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "B * L = %lld too large", (long long)B * L);

  relattn::DecodeArgs a;
  a.q = q; a.k = k_codes; a.v = v_codes; a.r = r; a.pc = P_cols; a.out = out; a.lse = lse;
  a.k_scale = k_scales; a.v_scale = v_scales;
  a.ws = static_cast<float*>(workspace);
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.d_r = rel_extent > 0 ? d_r : 16; a.E = rel_extent; a.W = window;
  const double s = paged ? 1.0 : scale_of(log_scale, L);  // paged: s per sequence on the device
  a.c1 = (float)(s * (double)alpha * 1.4426950408889634);
  a.c2 = (float)(s * 1.4426950408889634);
  a.n_split = pl.n_split;
  a.chunk = pl.chunk;
  a.kv_lo = pl.kv_lo;
  a.n_hg = pl.n_hg;
  a.rl_base = pl.rl_base;
  a.rl_stride = pl.rl_stride;
  a.rl = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.ws_partial_bytes);
  if (paged) {
    a.kv_len = kv_len; a.btab = block_table;
    a.max_pages = max_pages; a.num_pages = num_pages; a.page_size = page_size;
    a.log_scale = log_scale; a.alpha = alpha;
  }
  hipError_t e = relattn::launch_decode_mx(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rel_mx_quantize(const void* x, void* codes, void* scales, int dtype, long long n_rows, int D, void* stream) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_BF16 or RA_F32", dtype);
  if (n_rows < 0) return fail(RA_ERR_INVALID_ARG, "n_rows = %lld < 0", n_rows);
  if (D != relattn::kHeadDim) return fail(RA_ERR_UNSUPPORTED, "row length D = %d: only 128 is supported", D);
  if (n_rows == 0) return ok();
  int rc;
  if ((rc = check_ptr(x, "x", true)) || (rc = check_ptr(codes, "codes", true))) return rc;
  if (scales == nullptr) return fail(RA_ERR_INVALID_ARG, "scales is NULL");
  if (codes == x || scales == x) return fail(RA_ERR_INVALID_ARG, "an output aliases x");
  if (n_rows > 0x7fffffffLL * 16) return fail(RA_ERR_UNSUPPORTED, "n_rows = %lld too large", n_rows);
  hipError_t e = relattn::launch_mx_quantize(dtype, x, codes, scales, n_rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(e));
  return ok();
}

int rel_logits(const void* r, const void* P_cols, float* out, int dtype, long long n_tok, int H, int d_r,
               int rel_extent, int log_scale, long long seq_len, void* stream) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "dtype %d is not RA_BF16 or RA_F32", dtype);
  if (n_tok < 0 || H <= 0) return fail(RA_ERR_INVALID_ARG, "n_tok = %lld, H = %d", n_tok, H);
  if (rel_extent <= 0) return fail(RA_ERR_INVALID_ARG, "rel_extent = %d must be positive", rel_extent);
  if (log_scale != 0 && log_scale != 1) return fail(RA_ERR_INVALID_ARG, "log_scale = %d is not 0 or 1", log_scale);
  if (d_r <= 0 || d_r % 16 != 0 || d_r > relattn::kMaxDr)
    return fail(RA_ERR_UNSUPPORTED, "d_r = %d: supported values are multiples of 16 in [16, 128]", d_r);
  int rc;
  if ((rc = check_ptr(r, "r", true)) || (rc = check_ptr(P_cols, "P_cols", true)) || (rc = check_ptr(out, "out", true)))
    return rc;
  if (rel_extent > 65535 * 128) return fail(RA_ERR_UNSUPPORTED, "rel_extent = %d too large", rel_extent);
  if (n_tok == 0) return ok();
  relattn::RelLogitsArgs a;
  a.r = r; a.pc = P_cols; a.out = out;
  a.n_rows = n_tok * H;
  a.d_r = d_r; a.E = rel_extent;
  a.s = (float)scale_of(log_scale, seq_len);
  a.out_cols = rel_extent; a.out_stride = rel_extent; a.rev_base = 0;
  hipError_t e = relattn::launch_rel_logits(dtype, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "rel_logits launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
