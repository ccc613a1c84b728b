// Relative-attention decode for gfx950: one query token per sequence at
// position L-1 against a KV cache [B, L, Hkv, D].
//
// The logit is the one of page "SGLang and Miles Add Day-0 Support for
// Inkling", section "Attention with Relative Positional Embedding"; for the
// single query i = L-1 the bias of key j is s * r.P[:, L-1-j] when
// L-1-j < E.  The visible keys (all of them, or the last `window`) are cut
// into num_splits contiguous chunks ("num_splits" split-KV of the vLLM page,
// section on the sheared-bias FA4 kernel); each wave owns one (sequence, kv
// head, group of up to 16 query heads, split) and streams its chunk of K and
// V exactly once for every query head of the group.  The partial softmax
// states (unnormalised o, running max m, sum l) go to the caller's workspace
// and a second kernel merges them by log-sum-exp.
//
// Per 32-key step a wave computes S^T = K Q^T with 16x16x32 MFMAs (rows =
// keys, columns = query heads, padded to 16), adds the bias rows produced by
// R^T = P_rows r^T where each lane's A-operand row is the P row of its own
// key's distance (no shear is needed for a single query), applies the online
// softmax, and accumulates O^T = V^T P^T.  V is transposed through a
// wave-private LDS buffer.
#include "device_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecKeys = 32;  // keys per step

template <typename T>
struct DecodeCfg {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int VS = kDecKeys + PAD;  // V^T row stride (elements)
  static constexpr size_t LDS_WAVE = size_t(kHeadDim) * VS * sizeof(T);
};

// Slot of key kappa (0..31) in a V^T row: k-slot 8*g + t of the PV MFMA holds
// key 4*g + t (t < 4) or 16 + 4*g + (t-4) (t >= 4), the keys lane (g, c)
// holds in its two S^T accumulators.
__device__ __forceinline__ int dec_vt_pos(int kappa) {
  const int blk = kappa >> 4, r16 = kappa & 15;
  return 8 * (r16 >> 2) + 4 * blk + (r16 & 3);
}

// Write elements e of four consecutive keys' V vectors into one V^T row.
__device__ __forceinline__ void put4(__bf16* dst, const bf16x8 (&x)[8], int base, int e) {
  bf16x4 y;
  y[0] = x[base + 0][e];
  y[1] = x[base + 1][e];
  y[2] = x[base + 2][e];
  y[3] = x[base + 3][e];
  *reinterpret_cast<bf16x4*>(dst) = y;
}
__device__ __forceinline__ void put4(float* dst, const f32x8 (&x)[8], int base, int e) {
  f32x4 y;
  y[0] = x[base + 0][e];
  y[1] = x[base + 1][e];
  y[2] = x[base + 2][e];
  y[3] = x[base + 3][e];
  *reinterpret_cast<f32x4*>(dst) = y;
}

template <typename T>
__global__ __launch_bounds__(kDecWaves * 64) void decode_split_kernel(DecodeArgs p) {
  using C = DecodeCfg<T>;
  constexpr int D = kHeadDim;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kDecWaves * C::LDS_WAVE];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;   // lane group: k-slots 8g..8g+7, accumulator rows 4g..4g+3
  const int c = lane & 15;   // query head column / A-operand row

  const int L = p.L, Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const int d_r = p.d_r, E = p.E, W = p.W;

  // wave -> (batch, kv head, head group, split)
  const long long wid = (long long)blockIdx.x * kDecWaves + w;
  const long long n_waves = (long long)p.B * Hkv * p.n_hg * p.n_split;
  if (wid >= n_waves) return;
  const int split = (int)(wid % p.n_split);
  long long rest = wid / p.n_split;
  const int hg = (int)(rest % p.n_hg);
  rest /= p.n_hg;
  const int kvh = (int)(rest % Hkv);
  const int b = (int)(rest / Hkv);

  const int ks = p.kv_lo + split * p.chunk;
  const int ke = min(ks + p.chunk, L);

  const int hin = hg * 16 + c;  // head within the kv group
  const bool hvalid = hin < G;
  const int h = kvh * G + (hvalid ? hin : 0);

  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  const T* rg = static_cast<const T*>(p.r);
  const T* pcg = static_cast<const T*>(p.pc);

  // query (B operand of S^T = K Q^T): k-slot 8g+t of step st is d = 32*st + 8*g + t
  v8_t<T> qreg[D / 32];
#pragma unroll
  for (int st = 0; st < D / 32; ++st)
    qreg[st] = ld8_or_zero<T>(qg + (size_t(b) * Hq + h) * D + 32 * st + 8 * g, hvalid);
  v8_t<T> rreg[kMaxDr / 32];
#pragma unroll
  for (int st = 0; st < kMaxDr / 32; ++st) {
    const int c0 = 32 * st + 8 * g;
    rreg[st] = ld8_or_zero<T>(rg + (size_t(b) * Hq + h) * d_r + (c0 < d_r ? c0 : 0), E > 0 && hvalid && c0 < d_r);
  }
  const int nsr = (d_r + 31) / 32;

  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = zero4();
  float m_run = -INFINITY, l_run = 0.0f;

  T* vt = reinterpret_cast<T*>(smem + w * C::LDS_WAVE);
  const size_t row_stride = size_t(Hkv) * D;
  const T* kbase = kg + (size_t(b) * L * Hkv + kvh) * D;
  const T* vbase = vg + (size_t(b) * L * Hkv + kvh) * D;

  v8_t<T> kc[2][D / 32], vc[8];
  auto fetch = [&](int j0, v8_t<T> (&kd)[2][D / 32], v8_t<T> (&vd)[8]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int j = j0 + 16 * blk + c;
      const bool ok = j < ke;
      const T* src = kbase + size_t(ok ? j : ks) * row_stride + 8 * g;
#pragma unroll
      for (int st = 0; st < D / 32; ++st) kd[blk][st] = ld8_or_zero<T>(src + 32 * st, ok);
    }
    // V: lane (g, c) loads d-chunk c (8 values) of keys 8g .. 8g+7
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + 8 * g + i;
      const bool ok = j < ke;
      vd[i] = ld8_or_zero<T>(vbase + size_t(ok ? j : ks) * row_stride + 8 * c, ok);
    }
  };

  if (ks < ke) fetch(ks, kc, vc);
  for (int j0 = ks; j0 < ke; j0 += kDecKeys) {
    v8_t<T> kn[2][D / 32], vn[8];
    const bool more = j0 + kDecKeys < ke;
    if (more) fetch(j0 + kDecKeys, kn, vn);

    // scores: accumulator (blk, v) of lane (g, c) = key j0 + 16*blk + 4*g + v, head c
    f32x4 sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sc[blk] = zero4();
#pragma unroll
      for (int st = 0; st < D / 32; ++st) mma16(kc[blk][st], qreg[st], sc[blk]);
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[blk][v] *= p.c1;
    }

    // relative bias on keys with distance L-1-j < E
    if (E > 0 && (L - 1) - min(j0 + kDecKeys - 1, ke - 1) < E) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int j = j0 + 16 * blk + c;          // A-operand row of this lane
        const int dist = L - 1 - j;
        const bool ok = j < ke && dist >= 0 && dist < E;
        const T* prow = pcg + size_t(ok ? dist : 0) * d_r + 8 * g;
        f32x4 racc = zero4();
#pragma unroll
        for (int st = 0; st < kMaxDr / 32; ++st) {
          if (st < nsr) {
            const bool okc = ok && (32 * st + 8 * g) < d_r;
            mma16(ld8_or_zero<T>(prow + 32 * st, okc), rreg[st], racc);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[blk][v] += racc[v] * p.c2;
      }
    }

    // mask: past the split end, or outside the window
    const bool need_mask = (j0 + kDecKeys > ke) || (W > 0 && (L - 1) - j0 >= W);
    if (need_mask) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = j0 + 16 * blk + 4 * g + v;
          if (j >= ke || (W > 0 && (L - 1) - j >= W)) sc[blk][v] = -INFINITY;
        }
    }

    // online softmax per head (lanes c, c+16, c+32, c+48)
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
    v8_t<T> pb;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = fast_exp2(sc[blk][v] - m_use);
        psum += e;
        pb[4 * blk + v] = T(e);
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[i][v] *= corr;

    // V^T into LDS: V^T[d][slot] for d = 8c + e, keys 8g..8g+3 and 8g+4..8g+7
    {
      const int pos0 = dec_vt_pos(8 * g);
      const int pos1 = dec_vt_pos(8 * g + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        T* row = vt + (8 * c + e) * C::VS;
        put4(row + pos0, vc, 0, e);
        put4(row + pos1, vc, 4, e);
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int db = 0; db < D / 16; ++db) mma16(ld8<T>(vt + (16 * db + c) * C::VS + 8 * g), pb, o[db]);
    wave_lds_fence();

    if (more) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int st = 0; st < D / 32; ++st) kc[blk][st] = kn[blk][st];
#pragma unroll
      for (int i = 0; i < 8; ++i) vc[i] = vn[i];
    }
  }

  // partial state: sum l over the 4 lane groups; o rows d = 16*db + 4*g + v
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += xor_lane(l_tot, 32);
  if (!hvalid) return;
  const size_t n_bh = size_t(p.B) * Hq;
  const size_t bh = size_t(b) * Hq + h;
  float* ws_o = p.ws + (size_t(split) * n_bh + bh) * D;
  float* ws_m = p.ws + size_t(p.n_split) * n_bh * D;
  float* ws_l = ws_m + size_t(p.n_split) * n_bh;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(ws_o + 16 * db + 4 * g) = o[db];
  if (g == 0) {
    ws_m[size_t(split) * n_bh + bh] = m_run;
    ws_l[size_t(split) * n_bh + bh] = l_tot;
  }
}

// Log-sum-exp merge of the split partials: one workgroup per (batch, head),
// thread (sg, d4) covers splits sg, sg+8, ... and output columns 4*d4..4*d4+3.
constexpr int kMergeThreads = 256;

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs p) {
  constexpr int D = kHeadDim;
  constexpr int NSG = kMergeThreads / (D / 4);  // split groups (8)
  __shared__ float red_m[NSG];
  __shared__ float red_l[NSG][D / 4];
  __shared__ f32x4 red_o[NSG][D / 4];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int d4 = tid % (D / 4);
  const int sg = tid / (D / 4);
  const size_t n_bh = size_t(p.B) * p.Hq;
  const float* ws_o = p.ws;
  const float* ws_m = p.ws + size_t(p.n_split) * n_bh * D;
  const float* ws_l = ws_m + size_t(p.n_split) * n_bh;

  float mx = -INFINITY;
  for (int s = sg; s < p.n_split; s += NSG) mx = fmaxf(mx, ws_m[size_t(s) * n_bh + bh]);
  if (d4 == 0) red_m[sg] = mx;
  __syncthreads();
  float M = red_m[0];
#pragma unroll
  for (int i = 1; i < NSG; ++i) M = fmaxf(M, red_m[i]);
  const float Muse = (M == -INFINITY) ? 0.0f : M;

  f32x4 acc = zero4();
  float den = 0.0f;
  for (int s = sg; s < p.n_split; s += NSG) {
    const float wgt = fast_exp2(ws_m[size_t(s) * n_bh + bh] - Muse);
    const f32x4 os = *reinterpret_cast<const f32x4*>(ws_o + (size_t(s) * n_bh + bh) * D + 4 * d4);
    den += wgt * ws_l[size_t(s) * n_bh + bh];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += wgt * os[v];
  }
  red_o[sg][d4] = acc;
  red_l[sg][d4] = den;
  __syncthreads();
  if (sg != 0) return;
#pragma unroll
  for (int i = 1; i < NSG; ++i) {
    const f32x4 x = red_o[i][d4];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += x[v];
    den += red_l[i][d4];
  }
  const float inv = 1.0f / den;
  st4_f32<T>(static_cast<T*>(p.out) + size_t(bh) * D + 4 * d4, acc[0] * inv, acc[1] * inv, acc[2] * inv,
             acc[3] * inv);
  if (p.lse != nullptr && d4 == 0) p.lse[bh] = (Muse + log2f(den)) * kLn2;
}

template <typename T>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const long long n_waves = (long long)a.B * a.Hkv * a.n_hg * a.n_split;
  const long long grid = (n_waves + kDecWaves - 1) / kDecWaves;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_split_kernel<T>, dim3((unsigned)grid), dim3(kDecWaves * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<T>, dim3((unsigned)(a.B * a.Hq)), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int B, int L, int Hq, int Hkv, int num_splits_req, int window) {
  DecodePlan pl;
  const int G = Hq / Hkv;
  pl.n_hg = (G + 15) / 16;
  pl.kv_lo = (window > 0 && L > window) ? L - window : 0;
  const int vis = L - pl.kv_lo;
  const int max_split = (vis + kDecKeys - 1) / kDecKeys;  // at least one 32-key step per split
  int ns;
  if (num_splits_req > 0) {
    ns = num_splits_req;
  } else {
    // Aim for ~1024 waves (4 per CU of a 256-CU part) and at least 256 keys per split.
    const long long waves_per_split = (long long)B * Hkv * pl.n_hg;
    long long want = (1024 + waves_per_split - 1) / waves_per_split;
    const long long cap = (vis + 255) / 256;
    if (want > cap) want = cap;
    ns = (int)(want < 1 ? 1 : want);
  }
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  int chunk = (vis + ns - 1) / ns;
  chunk = (chunk + kDecKeys - 1) / kDecKeys * kDecKeys;
  ns = (vis + chunk - 1) / chunk;  // drop splits that would be empty
  if (ns < 1) ns = 1;
  pl.n_split = ns;
  pl.chunk = chunk < kDecKeys ? kDecKeys : chunk;
  const size_t n_bh = size_t(B) * Hq;
  pl.ws_bytes = size_t(ns) * n_bh * (kHeadDim + 2) * sizeof(float);
  return pl;
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_decode_t<__bf16>(a, stream);
  return launch_decode_t<float>(a, stream);
}

}  // namespace relattn
