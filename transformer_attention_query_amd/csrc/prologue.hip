// The attention prologue for gfx950: K/V ShortConv, Q/K RMSNorm and the
// KV-cache write in one pass over the new tokens' projections (page "SGLang
// and Miles Add Day-0 Support for Inkling", section "ShortConv
// Optimization", paragraph "KV ShortConv + QK-norm + KV store"; the filter is
// the equation of section "Short Convolution (ShortConv)",
// y[t,c] = x[t,c] + sum_{d<W} w[c,d] * x[t-d,c]).
//
// Work decomposition.  The new rows are packed by sequence.  A head unit is
// one head's D = 128 channels of one token's q, k or v row: Hq + 2*Hkv units
// per token.  Sixteen lanes own one unit, eight channels each (one 16-byte
// bf16 vector), and walk a block of TB consecutive packed tokens:
//   * q units: y = x * rsqrt(mean(x^2) + eps) * g_q, written to q_out;
//   * k units: the ShortConv (the three previous raw rows kept in registers),
//     then the RMSNorm with g_k, written to the k cache at the token's
//     position;
//   * v units: the ShortConv, written to the v cache.
// The mean over a head's channels is a 16-lane sum: DPP row rotations by 8,
// 4, 2 and 1.  Arithmetic is fp32; the residual is added after the filter
// taps, and each output is rounded once.  At a sequence's first new token the
// previous rows come from the caller's state (or zeros); the unit that handles
// a sequence's last new token writes its three last raw rows to the new
// state.  Extra units copy the state of sequences with no new token.
//
// Memory: one read of every q, k and v row (plus three rows before each token
// block for the filter, usually L2 hits) and one write of every output row --
// the kernel is bound by HBM bandwidth.
#include "device_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr int kTB = 16;         // tokens per unit
constexpr int kStateRows = 3;   // raw rows kept per stream and sequence
constexpr int kSeqLds = 4096;   // sequence offsets staged in LDS up to this many

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&x)[8]) {
  const v8_t<T> v = ld8<T>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = float(v[i]);
}
template <typename T>
__device__ __forceinline__ void store8f(T* p, const float (&x)[8]) {
  v8_t<T> v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = T(x[i]);
  st8<T>(p, v);
}

// Sum over the 16 lanes of a DPP row; every lane gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs p, int n_blocks, int n_units) {
  __shared__ int s_qs[kSeqLds];
  const int B = p.B;
  const bool seq_in_lds = B + 1 <= kSeqLds;
  if (seq_in_lds)
    for (int i = threadIdx.x; i <= B; i += blockDim.x) s_qs[i] = p.q_start[i];
  __syncthreads();
  // packed row offsets, clamped to [0, total_q] so any contents keep every access in bounds
  auto qs = [&](int b) { return min(max(seq_in_lds ? s_qs[b] : p.q_start[b], 0), p.total_q); };

  const int lane16 = threadIdx.x & 15;
  const int unit = blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4);
  const int Hq = p.Hq, Hkv = p.Hkv, U = Hq + 2 * Hkv;
  const int C = Hkv * kHeadDim;
  if (unit >= n_units) return;
  const int c0 = 8 * lane16;  // this lane's channels within the head

  // ---- state copy of a sequence with no new token
  if (unit >= n_blocks * U) {
    const int cu = unit - n_blocks * U;  // (b, stream, kv head)
    const int b = cu / (2 * Hkv), s = (cu / Hkv) % 2, hk = cu % Hkv;
    if (p.state_out == nullptr || qs(b + 1) != qs(b)) return;
    T* so = static_cast<T*>(p.state_out) + (size_t(b) * 2 + s) * kStateRows * C + hk * kHeadDim + c0;
    const T* si = p.state_in ? static_cast<const T*>(p.state_in) + (size_t(b) * 2 + s) * kStateRows * C +
                                    hk * kHeadDim + c0
                             : nullptr;
#pragma unroll
    for (int j = 0; j < kStateRows; ++j) {
      float x[8];
      if (si) load8f<T>(si + j * C, x);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.0f;
      store8f<T>(so + j * C, x);
    }
    return;
  }

  const int blk = unit / U, hu = unit % U;
  const int t0 = blk * kTB;
  const int t1 = min(t0 + kTB, p.total_q);
  const float eps = p.eps;

  // ---- q units: RMSNorm only
  if (hu < Hq) {
    float g[8];
    load8f<T>(static_cast<const T*>(p.q_norm_w) + c0, g);
    const T* qi = static_cast<const T*>(p.q_in) + size_t(hu) * kHeadDim + c0;
    T* qo = static_cast<T*>(p.q_out) + size_t(hu) * kHeadDim + c0;
    const size_t rs = size_t(Hq) * kHeadDim;
    v8_t<T> xr[kTB];  // raw rows, converted on use (half the registers for bf16)
#pragma unroll
    for (int i = 0; i < kTB; ++i)
      if (t0 + i < t1) xr[i] = ld8<T>(qi + size_t(t0 + i) * rs);
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      if (t0 + i >= t1) break;
      float xt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xt[e] = float(xr[i][e]);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xt[e], xt[e], ss);
      const float inv = rsqrtf(row16_sum(ss) * (1.0f / kHeadDim) + eps);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = xt[e] * inv * g[e];
      store8f<T>(qo + size_t(t0 + i) * rs, y);
    }
    return;
  }

  // ---- k and v units: ShortConv (+ RMSNorm for k) and the cache write
  const bool is_k = hu < Hq + Hkv;
  const int hk = is_k ? hu - Hq : hu - Hq - Hkv;
  const int s = is_k ? 0 : 1;
  const T* xin = static_cast<const T*>(is_k ? p.k_in : p.v_in) + size_t(hk) * kHeadDim + c0;
  const size_t rs = size_t(Hkv) * kHeadDim;
  T* cache = static_cast<T*>(is_k ? p.k_cache : p.v_cache);
  const int W = p.conv_w;
  float wt[4][8];  // wt[d][e] = w[channel, d]
  {
    const T* wp = static_cast<const T*>(is_k ? p.conv_k : p.conv_v) + (size_t(hk) * kHeadDim + c0) * W;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int d = 0; d < 4; ++d) wt[d][e] = d < W ? float(wp[e * W + d]) : 0.0f;
  }
  float g[8];
  if (is_k) load8f<T>(static_cast<const T*>(p.k_norm_w) + c0, g);

  v8_t<T> xr[kTB];  // raw rows, converted on use
#pragma unroll
  for (int i = 0; i < kTB; ++i)
    if (t0 + i < t1) xr[i] = ld8<T>(xin + size_t(t0 + i) * rs);

  // Sequence tracking: b is the last sequence whose first row is <= t0; the
  // walk moves forward over empty sequences.  A token that lies in no
  // sequence (possible only with inconsistent offsets) is skipped.
  int b;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qs(mid) <= t0) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }
  int sb = qs(b), se = qs(b + 1);
  const T* st_in = static_cast<const T*>(p.state_in);
  T* st_out = static_cast<T*>(p.state_out);
  auto state_row = [&](int j, float (&r)[8]) {  // raw row j (0 = oldest) before sequence b's chunk
    if (st_in) load8f<T>(st_in + ((size_t(b) * 2 + s) * kStateRows + j) * C + hk * kHeadDim + c0, r);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = 0.0f;
  };
  // previous raw rows: w1 = x[t-1], w2 = x[t-2], w3 = x[t-3]
  float w1[8], w2[8], w3[8];
  auto prev_row = [&](int t, int i, int d, float (&r)[8]) {  // raw row of position i - d before token t
    if (i - d >= 0) load8f<T>(xin + size_t(t - d) * rs, r);
    else state_row(kStateRows + i - d, r);
  };
  auto init_window = [&](int t) {
    const int i = t - sb;  // 0 <= i: position of t within the chunk
    prev_row(t, i, 1, w1);
    prev_row(t, i, 2, w2);
    prev_row(t, i, 3, w3);
  };
  bool need_init = true;
  int pos0 = 0;  // cache position of the sequence's first new row
  const int* btab = p.btab;

#pragma unroll
  for (int i = 0; i < kTB; ++i) {
    const int t = t0 + i;
    if (t >= t1) break;
    if (t >= se) {
      while (t >= se && b < B - 1) {
        ++b;
        sb = se;
        se = qs(b + 1);
      }
      need_init = true;
    }
    if (t < sb || t >= se) continue;
    if (need_init) {  // first token of this unit in sequence b: the window comes from the rows before it
      init_window(t);
      pos0 = p.kv_len[b] - (se - sb);
      need_init = false;
    }
    float xt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xt[e] = float(xr[i][e]);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = wt[0][e] * xt[e];
      acc = fmaf(wt[1][e], w1[e], acc);
      acc = fmaf(wt[2][e], w2[e], acc);
      acc = fmaf(wt[3][e], w3[e], acc);
      y[e] = acc + xt[e];
    }
    if (is_k) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
      const float inv = rsqrtf(row16_sum(ss) * (1.0f / kHeadDim) + eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = y[e] * inv * g[e];
    }
    // cache write at the token's position; rows outside the cache are skipped
    const int pos = pos0 + (t - sb);
    long long row = -1;
    if (btab == nullptr) {
      if (pos >= 0 && pos < p.cap) row = (long long)b * p.cap + pos;
    } else if (pos >= 0 && pos < p.max_pages * p.page_size) {
      const int pg = btab[size_t(b) * p.max_pages + pos / p.page_size];
      if (pg >= 0 && pg < p.num_pages) row = (long long)pg * p.page_size + pos % p.page_size;
    }
    if (row >= 0) store8f<T>(cache + size_t(row) * rs + size_t(hk) * kHeadDim + c0, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w3[e] = w2[e];
      w2[e] = w1[e];
      w1[e] = xt[e];
    }
    if (t == se - 1 && st_out != nullptr) {  // last new token: its three last raw rows are the new state
      T* so = st_out + (size_t(b) * 2 + s) * kStateRows * C + hk * kHeadDim + c0;
      store8f<T>(so, w3);
      store8f<T>(so + C, w2);
      store8f<T>(so + 2 * C, w1);
    }
  }
}

template <typename T>
hipError_t launch_t(const PrologueArgs& a, hipStream_t stream) {
  const long long n_blocks = (a.total_q + kTB - 1) / kTB;
  const long long U = a.Hq + 2LL * a.Hkv;
  const long long n_units = n_blocks * U + (long long)a.B * 2 * a.Hkv;
  if (n_units > 0x7fffffffLL - 16) return hipErrorInvalidConfiguration;
  const long long grid = (n_units + 15) / 16;
  hipLaunchKernelGGL(prologue_kernel<T>, dim3((unsigned)grid), dim3(256), 0, stream, a, (int)n_blocks,
                     (int)n_units);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(int dtype, const PrologueArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_t<__bf16>(a, stream);
  return launch_t<float>(a, stream);
}

}  // namespace relattn
