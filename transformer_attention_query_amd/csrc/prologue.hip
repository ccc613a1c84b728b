// The attention prologue for gfx950: K/V ShortConv, Q/K RMSNorm and the
// KV-cache write in one pass over the new tokens' projections (page "SGLang
// and Miles Add Day-0 Support for Inkling", section "ShortConv
// Optimization", paragraph "KV ShortConv + QK-norm + KV store"; the filter is
// the equation of section "Short Convolution (ShortConv)",
// y[t,c] = x[t,c] + sum_{d<W} w[c,d] * x[t-d,c]).
//
// Work decomposition: one launch whose workgroups do one of two jobs.
//   * q rows: y = x * rsqrt(mean(x^2) + eps) * g_q for every q row
//     (token, head).  Sixteen lanes own one row of D = 128 channels, eight
//     each (one 16-byte bf16 vector), and a group takes four consecutive
//     rows, so a wave streams contiguous memory; no sequence lookup is needed.
//   * k and v rows (the first workgroups).  Sixteen lanes own one kv head of k
//     or v over a block of four tokens and load the block's raw rows with the
//     three before it at once (rows before the sequence's chunk come from the
//     caller's state, or are zeros): the ShortConv, then (k) the RMSNorm with
//     g_k, then the write to the cache at each token's position.  The group
//     of a sequence's last new token writes its three last raw rows to the
//     new state.  Extra groups copy the state of sequences with no new token.
// The mean over a head's channels is a 16-lane sum: DPP row rotations by 8,
// 4, 2 and 1.  Arithmetic is fp32; the residual is added after the filter
// taps, and each output is rounded once.
//
// Memory: one read of every q, k and v row (the filter's re-reads of the
// three previous k / v rows hit the caches) and one write of every output
// row -- the kernels are bound by HBM bandwidth.
#include "device_common.hpp"
#include "mx_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr int kStateRows = 3;   // raw rows kept per stream and sequence
constexpr int kSeqLds = 2048;   // sequence offsets and lengths staged in LDS up to this many

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

// q rows: RMSNorm only.  A 16-lane group normalises kQRows consecutive
// (token, head) rows of q (the packed rows are one flat array of heads), so a
// wave streams 4 * kQRows * 256 contiguous bytes with no sequence lookup.
constexpr int kQRows = 4;

template <typename T>
__device__ __forceinline__ void q_rows(const PrologueArgs& p, int wg, long long n_rows) {
  const int lane16 = threadIdx.x & 15;
  const long long g = (long long)wg * 16 + (threadIdx.x >> 4);
  const long long r0 = g * kQRows;
  if (r0 >= n_rows) return;
  const int c0 = 8 * lane16;
  const T* qi = static_cast<const T*>(p.q_in) + c0;
  T* qo = static_cast<T*>(p.q_out) + c0;
  v8_t<T> xr[kQRows];
#pragma unroll
  for (int k = 0; k < kQRows; ++k) xr[k] = ld8<T>(qi + size_t(min(r0 + k, n_rows - 1)) * kHeadDim);
  float gw[8];
  load8f<T>(static_cast<const T*>(p.q_norm_w) + c0, gw);
#pragma unroll
  for (int k = 0; k < kQRows; ++k) {
    if (r0 + k >= n_rows) break;
    float xt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xt[e] = float(xr[k][e]);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(xt[e], xt[e], ss);
    const float inv = rsqrtf(row16_sum(ss) * (1.0f / kHeadDim) + p.eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = xt[e] * inv * gw[e];
    store8f<T>(qo + size_t(r0 + k) * kHeadDim, y);
  }
}

// k and v rows: ShortConv, RMSNorm for k, cache write, state.  One 16-lane
// group per (block of kTB tokens, k or v, kv head): it loads the block's raw
// rows and the three before it in one go (neighbouring groups re-read those
// three, which hit the caches), loads the filter taps once, and produces the
// block's rows; rows before a sequence's chunk come from the state.
constexpr int kTB = 4;

template <typename T, bool MX>
__device__ __forceinline__ void kv_rows(const PrologueArgs& p, int wg, int n_row_units, int n_units) {
  __shared__ int s_qs[kSeqLds];
  __shared__ int s_kv[kSeqLds];
  const int B = p.B;
  const bool seq_in_lds = B + 1 <= kSeqLds;
  if (seq_in_lds)
    for (int i = threadIdx.x; i <= B; i += blockDim.x) {
      s_qs[i] = p.q_start[i];
      if (i < B) s_kv[i] = p.kv_len[i];
    }
  __syncthreads();
  // packed row offsets, clamped to [0, total_q] so any contents keep every access in bounds
  auto qs = [&](int b) { return min(max(seq_in_lds ? s_qs[b] : p.q_start[b], 0), p.total_q); };

  const int lane16 = threadIdx.x & 15;
  const int unit = wg * (blockDim.x / 16) + (threadIdx.x >> 4);
  const int Hkv = p.Hkv, U = 2 * Hkv;  // per token block: k heads, then v heads
  const int C = Hkv * kHeadDim;
  if (unit >= n_units) return;
  const int c0 = 8 * lane16;  // this lane's channels within the head

  // ---- state copy of a sequence with no new token
  if (unit >= n_row_units) {
    const int cu = unit - n_row_units;  // (b, stream, kv head)
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

  const int blk = unit / U, su = unit % U;
  const bool is_k = su < Hkv;
  const int hk = is_k ? su : su - Hkv;
  const int s = is_k ? 0 : 1;
  const int t0 = blk * kTB;
  const int t1 = min(t0 + kTB, p.total_q);
  const T* xin = static_cast<const T*>(is_k ? p.k_in : p.v_in) + size_t(hk) * kHeadDim + c0;
  const size_t rs = size_t(Hkv) * kHeadDim;
  // xr[j] = raw row t0 - 3 + j (clamped into [0, t1)); rows before the
  // sequence's chunk are replaced by state rows below
  v8_t<T> xr[kTB + 3];
#pragma unroll
  for (int j = 0; j < kTB + 3; ++j) xr[j] = ld8<T>(xin + size_t(min(max(t0 - 3 + j, 0), t1 - 1)) * rs);
  const int W = p.conv_w;
  float wt[4][8];  // wt[d][e] = w[channel, d]
  {
    const T* wp = static_cast<const T*>(is_k ? p.conv_k : p.conv_v) + (size_t(hk) * kHeadDim + c0) * W;
    if (W == 4 && (reinterpret_cast<uintptr_t>(wp) & 15) == 0) {
      // the lane's 8 channels x 4 taps are 32 contiguous values: four vectors
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const v8_t<T> wv = ld8<T>(wp + 8 * v);
#pragma unroll
        for (int k = 0; k < 8; ++k) wt[k % 4][2 * v + k / 4] = float(wv[k]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int d = 0; d < 4; ++d) wt[d][e] = d < W ? float(wp[e * W + d]) : 0.0f;
    }
  }
  float g[8];
  if (is_k) load8f<T>(static_cast<const T*>(p.k_norm_w) + c0, g);

  // sequence of token t0: the last b whose first row is <= t0
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
#pragma unroll
  for (int k = 0; k < kTB; ++k) {
    const int t = t0 + k;
    if (t >= t1) break;
    while (t >= se && b < B - 1) {  // the next sequence (over empty ones)
      ++b;
      sb = se;
      se = qs(b + 1);
    }
    if (t < sb || t >= se) continue;  // a token in no sequence (inconsistent offsets)
    const int i = t - sb;             // position of t within the chunk
    float x[4][8];                    // x[d] = raw row t - d
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (i - d >= 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[d][e] = float(xr[k + 3 - d][e]);
      } else if (p.state_in != nullptr) {
        load8f<T>(static_cast<const T*>(p.state_in) + ((size_t(b) * 2 + s) * kStateRows + kStateRows + i - d) * C +
                      hk * kHeadDim + c0,
                  x[d]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[d][e] = 0.0f;
      }
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = wt[0][e] * x[0][e];
      acc = fmaf(wt[1][e], x[1][e], acc);
      acc = fmaf(wt[2][e], x[2][e], acc);
      acc = fmaf(wt[3][e], x[3][e], acc);
      y[e] = acc + x[0][e];
    }
    if (is_k) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
      const float inv = rsqrtf(row16_sum(ss) * (1.0f / kHeadDim) + p.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = y[e] * inv * g[e];
    }
    // cache write at the token's position; rows outside the cache are skipped
    const int pos = (seq_in_lds ? s_kv[b] : p.kv_len[b]) - (se - sb) + i;
    long long row = -1;
    if (p.btab == nullptr) {
      if (pos >= 0 && pos < p.cap) row = (long long)b * p.cap + pos;
    } else if (pos >= 0 && pos < p.max_pages * p.page_size) {
      const int pg = p.btab[size_t(b) * p.max_pages + pos / p.page_size];
      if (pg >= 0 && pg < p.num_pages) row = (long long)pg * p.page_size + pos % p.page_size;
    }
    if constexpr (MX) {
      // E4M3 codes with the scale of the 32-channel block (the lane's quad)
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
      const int sh = mx_shared_exp(quad_max(amax));
      uint2 cw;
      cw.x = e4m3_pack4(y[0], y[1], y[2], y[3], sh);
      cw.y = e4m3_pack4(y[4], y[5], y[6], y[7], sh);
      if (row >= 0) {
        unsigned char* cc = static_cast<unsigned char*>(is_k ? p.k_cache : p.v_cache);
        unsigned char* sc = static_cast<unsigned char*>(is_k ? p.k_scale : p.v_scale);
        *reinterpret_cast<uint2*>(cc + (size_t(row) * Hkv + hk) * kHeadDim + c0) = cw;
        if ((lane16 & 3) == 0)
          sc[(size_t(row) * Hkv + hk) * (kHeadDim / kMxBlock) + (lane16 >> 2)] = (unsigned char)(sh + 127);
      }
    } else {
      T* cache = static_cast<T*>(is_k ? p.k_cache : p.v_cache);
      if (row >= 0) store8f<T>(cache + size_t(row) * rs + size_t(hk) * kHeadDim + c0, y);
    }
    if (t == se - 1 && p.state_out != nullptr) {  // last new token: its three last raw rows are the new state
      T* so = static_cast<T*>(p.state_out) + (size_t(b) * 2 + s) * kStateRows * C + hk * kHeadDim + c0;
      store8f<T>(so, x[2]);
      store8f<T>(so + C, x[1]);
      store8f<T>(so + 2 * C, x[0]);
    }
  }
}

// One launch for both jobs: the k / v workgroups come first (they start
// first and their latency-bound work overlaps the q rows' streaming).
template <typename T, bool MX = false>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs p, int n_kv_wg, int n_row_units, int n_units,
                                                       long long n_q) {
  if ((int)blockIdx.x < n_kv_wg) kv_rows<T, MX>(p, blockIdx.x, n_row_units, n_units);
  else q_rows<T>(p, blockIdx.x - n_kv_wg, n_q);
}

template <typename T, bool MX = false>
hipError_t launch_t(const PrologueArgs& a, hipStream_t stream) {
  const long long n_q = (long long)a.total_q * a.Hq;
  const long long q_wg = (n_q + 16 * kQRows - 1) / (16 * kQRows);
  const long long n_rows = (a.total_q + kTB - 1) / kTB * 2LL * a.Hkv;
  const long long n_units = n_rows + (long long)a.B * 2 * a.Hkv;
  const long long kv_wg = (n_units + 15) / 16;
  if (n_units > 0x7fffffffLL - 16 || q_wg + kv_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prologue_kernel<T, MX>), dim3((unsigned)(q_wg + kv_wg)), dim3(256), 0, stream, a, (int)kv_wg,
                     (int)n_rows, (int)n_units, n_q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue_mx(const PrologueArgs& a, hipStream_t stream) { return launch_t<__bf16, true>(a, stream); }

hipError_t launch_prologue(int dtype, const PrologueArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_t<__bf16>(a, stream);
  return launch_t<float>(a, stream);
}

}  // namespace relattn
