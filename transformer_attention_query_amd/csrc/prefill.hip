// Relative-attention prefill for gfx950.
//
// Computes, for every query i of a sequence and query head h (page "SGLang
// and Miles Add Day-0 Support for Inkling", section "Attention with Relative
// Positional Embedding", eqs. for rel_logits and l(i,j,h)):
//   l(i,j) = s*alpha*q_i.k_j + [0 <= i-j < E] * s * r_i.P[:, i-j]
// under the causal / sliding-window mask, then the softmax over j and the
// weighted sum of v_j, in one pass (online softmax, the bias added before the
// running max as the FA4 fork does -- section "Relative Logits
// Optimization", Figure 3).
//
// Work decomposition
//   * One workgroup = WAVES waves = M = 32*WAVES consecutive queries of one
//     (batch, query head); it walks the key tiles of N keys that the mask
//     leaves visible (tiles entirely in the future or entirely outside the
//     window are never touched).
//   * Scores are computed transposed, S^T = K Q^T, so lane l of a wave owns
//     query l%32 and the 32x32 MFMA accumulators run over keys: the row max
//     and row sum are in-lane reductions plus one exchange with lane l^32,
//     and the output accumulator O^T = V^T P^T needs no cross-lane traffic
//     for its rescaling.
//   * K tiles are staged in LDS row-major, V tiles transposed (d-major, with
//     the keys of each 16-key chunk permuted so that one 16-byte LDS read
//     yields the 8 keys a lane feeds to the PV MFMA).
//   * Relative bias ("sheared bias" of section "Relative Logits
//     Optimization": bias(i,j) = rel_logits(i, i-j)) is formed per wave in
//     LDS: the wave's tile needs distances in [i0w - j0 - N + 1, i0w - j0 + 31];
//     it computes R^T = P_rows r^T for those N+32 distances with MFMA (P rows
//     staged in LDS for the whole workgroup), writes R into a wave-private LDS
//     buffer indexed [query][distance], and reads it back along the shear
//     (row a, column a - b + N for key b) -- a lane only ever reads its own
//     query's row.  Distances outside [0, E) read zero rows of P, so the
//     rel_extent cut and the causal edge need no per-score test.
//   * K/V for the next tile are fetched into registers while the current
//     tile computes.
#include "device_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

template <typename T, int WAVES, int N>
struct PrefillCfg {
  static constexpr int M = 32 * WAVES;       // queries per workgroup
  static constexpr int NB = N / 32;          // 32-key blocks per tile
  static constexpr int PAD = 16 / sizeof(T); // 16 bytes of padding per LDS row
  static constexpr int KS = kHeadDim + PAD;  // K tile row stride (elements)
  static constexpr int VS = N + PAD;         // V^T tile row stride
  static constexpr int PSMAX = kMaxDr + PAD; // P slice row stride (max)
  static constexpr int NR = M + N;           // P slice rows (distances)
  static constexpr int LS = N + 36;          // R buffer row stride (floats)
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KV_VECS = N * (kHeadDim / 8) / THREADS;  // 8-element vectors per thread per tile
  static constexpr size_t LDS_K = size_t(N) * KS * sizeof(T);
  static constexpr size_t LDS_V = size_t(kHeadDim) * VS * sizeof(T);
  static constexpr size_t LDS_P = size_t(NR) * PSMAX * sizeof(T);
  static constexpr size_t LDS_R = size_t(WAVES) * 32 * LS * sizeof(float);
  static constexpr size_t LDS_TOTAL = LDS_K + LDS_V + LDS_P + LDS_R;
  static_assert(KV_VECS * THREADS == N * (kHeadDim / 8), "tile must split evenly over threads");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// Position of key `row` (0..N-1) inside a V^T row: within each 16-key chunk
// the middle two groups of four are swapped, so that k-slot 8*h + t of the
// PV MFMA (h = lane/32) holds key 8*(t/4) + 4*h + t%4, which is the key the
// S^T accumulator register 8*(chunk%2) + t of that lane holds.
__device__ __forceinline__ int vt_pos(int row) {
  int k16 = row & 15;
  int p16 = ((k16 >> 2) & 1) * 8 + (k16 >> 3) * 4 + (k16 & 3);
  return (row & ~15) + p16;
}

template <typename T, int WAVES, int N>
__global__ __launch_bounds__(WAVES * 64, 1) void prefill_kernel(PrefillArgs p, int n_qt, int n_groups) {
  using C = PrefillCfg<T, WAVES, N>;
  constexpr int M = C::M, NB = C::NB;
  constexpr int D = kHeadDim;

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_TOTAL];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = reinterpret_cast<T*>(smem + C::LDS_K);
  T* Pt = reinterpret_cast<T*>(smem + C::LDS_K + C::LDS_V);
  float* Rs = reinterpret_cast<float*>(smem + C::LDS_K + C::LDS_V + C::LDS_P);

  const int T_ = p.T, Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const int d_r = p.d_r, E = p.E, W = p.W;

  // ---- workgroup -> (q-tile, batch, kv head, query head)
  // Workgroup ids reach the 8 XCDs round-robin.  Groups of G workgroups (the
  // query heads sharing one kv head, same q-tile) are placed on one XCD so
  // their K/V tiles are shared through that XCD's L2; groups are ordered
  // longest-first (late q-tiles see the most keys under the causal mask).
  const int pid = blockIdx.x;
  const int xcd = pid & 7;
  const int slot = pid >> 3;
  const int gi = (slot / G) * 8 + xcd;
  if (gi >= n_groups) return;
  const int member = slot % G;
  const int BH = p.B * Hkv;
  const int qt = n_qt - 1 - gi / BH;
  const int bk = gi % BH;
  const int b = bk / Hkv;
  const int kvh = bk % Hkv;
  const int h = kvh * G + member;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;  // half-wave
  const int a = lane & 31;   // this lane's query within the wave

  const int i0 = qt * M;
  const int qw0 = i0 + 32 * w;
  const int qa = qw0 + a;
  const bool qvalid = qa < T_;

  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  const T* rg = static_cast<const T*>(p.r);
  const T* pcg = static_cast<const T*>(p.pc);

  // ---- this lane's query and relative feature, as MFMA B operands
  v8_t<T> qreg[D / 16];
  {
    const T* qrow = qg + ((size_t(b) * T_ + (qvalid ? qa : 0)) * Hq + h) * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = ld8_or_zero<T>(qrow + kk * 16, qvalid);
  }
  v8_t<T> rreg[kMaxDr / 16];
  const int nkr = d_r / 16;
  if (E > 0) {
    const T* rrow = rg + ((size_t(b) * T_ + (qvalid ? qa : 0)) * Hq + h) * d_r + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) rreg[kk] = ld8_or_zero<T>(rrow + kk * 16, qvalid && kk < nkr);
  } else {
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) rreg[kk] = zero8<T>();
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // ---- visible key tiles of this q-tile
  const int i_last = min(i0 + M - 1, T_ - 1);
  int kt_lo = 0;
  if (W > 0) kt_lo = max(0, i0 - W + 1) / N;
  const int kt_hi = i_last / N;

  // ---- register prefetch of one K/V tile
  v8_t<T> kpre[C::KV_VECS], vpre[C::KV_VECS];
  const size_t kv_row_stride = size_t(Hkv) * D;
  const T* kbase = kg + (size_t(b) * T_ * Hkv + kvh) * D;
  const T* vbase = vg + (size_t(b) * T_ * Hkv + kvh) * D;
  auto fetch_kv = [&](int kt) {
    const int j0 = kt * N;
#pragma unroll
    for (int i = 0; i < C::KV_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      const int row = vid >> 4, c8 = vid & 15;
      const int j = j0 + row;
      const bool ok = j < T_;
      const size_t off = size_t(ok ? j : 0) * kv_row_stride + c8 * 8;
      kpre[i] = ld8_or_zero<T>(kbase + off, ok);
      vpre[i] = ld8_or_zero<T>(vbase + off, ok);
    }
  };

  fetch_kv(kt_lo);

  const int PS = d_r + C::PAD;
  float* rs = Rs + w * 32 * C::LS;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * N;
    const int D0 = i0 - j0;  // distance between the first query and the first key of the tile
    const bool wg_band = E > 0 && max(0, D0 - (N - 1)) < E;

    __syncthreads();  // every wave is done reading the previous tile
    // K row-major, V transposed with the PV key permutation
#pragma unroll
    for (int i = 0; i < C::KV_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      const int row = vid >> 4, c8 = vid & 15;
      st8<T>(Ks + row * C::KS + c8 * 8, kpre[i]);
      const int pos = vt_pos(row);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(c8 * 8 + e) * C::VS + pos] = vpre[i][e];
    }
    if (wg_band) {
      // P rows for distances D0 - N .. D0 + M - 1 (zero outside [0, E))
      const int vec_per_row = d_r / 8;
      const int nvec = C::NR * vec_per_row;
      for (int vid = tid; vid < nvec; vid += C::THREADS) {
        const int rho = vid / vec_per_row, c8 = vid - rho * vec_per_row;
        const int d = D0 - N + rho;
        const bool ok = d >= 0 && d < E;
        st8<T>(Pt + rho * PS + c8 * 8, ld8_or_zero<T>(pcg + size_t(ok ? d : 0) * d_r + c8 * 8, ok));
      }
    }
    __syncthreads();

    if (kt < kt_hi) fetch_kv(kt + 1);

    // ---- per-wave work on the (32 queries) x (N keys) sub-tile
    const bool wdead = qw0 >= T_ || j0 > qw0 + 31 || (W > 0 && qw0 - (j0 + N - 1) >= W);
    if (wdead) continue;
    const bool wband = E > 0 && max(0, qw0 - (j0 + N - 1)) < E;
    const bool wmask = (j0 + N - 1 > qw0) || (W > 0 && qw0 + 31 - j0 >= W);

    // S^T = K Q^T
    f32x16 s[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = zero16();
      const T* krow = Ks + (nb * 32 + a) * C::KS + 8 * h2;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) mma32(ld8<T>(krow + kk * 16), qreg[kk], s[nb]);
    }

    // logits in base 2: t = c1 * q.k (+ c2 * r.P on the sheared distance)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[nb][v] *= p.c1;

    if (wband) {
      // R^T for this wave's N+32 distances: rows 32*w + rb*32 + (0..31) of the P slice
#pragma unroll
      for (int rb = 0; rb <= NB; ++rb) {
        f32x16 racc = zero16();
        const T* prow = Pt + (32 * w + rb * 32 + a) * PS + 8 * h2;
#pragma unroll
        for (int kk = 0; kk < kMaxDr / 16; ++kk)
          if (kk < nkr) mma32(ld8<T>(prow + kk * 16), rreg[kk], racc);
        float* dst = rs + a * C::LS + rb * 32 + 4 * h2;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 x;
          x[0] = racc[4 * g4 + 0] * p.c2;
          x[1] = racc[4 * g4 + 1] * p.c2;
          x[2] = racc[4 * g4 + 2] * p.c2;
          x[3] = racc[4 * g4 + 3] * p.c2;
          *reinterpret_cast<f32x4*>(dst + g4 * 8) = x;
        }
      }
      wave_lds_fence();
      // key b of accumulator (nb, v): nb*32 + 8*(v/4) + 4*h2 + v%4; its distance column is a - b + N
      const float* src = rs + a * C::LS + a + N - 4 * h2;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[nb][v] += src[-(nb * 32 + 8 * (v >> 2) + (v & 3))];
      wave_lds_fence();
    }

    if (wmask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + nb * 32 + 8 * (v >> 2) + 4 * h2 + (v & 3);
          const int dd = qa - j;
          const bool vis = dd >= 0 && (W == 0 || dd < W);
          if (!vis) s[nb][v] = -INFINITY;
        }
    }

    // online softmax (per query = per lane pair l, l^32)
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[nb][v]);
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(s[nb][v] - m_use);
        s[nb][v] = e;
        psum += e;
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][v] *= corr;

    // O^T += V^T P^T
#pragma unroll
    for (int c16 = 0; c16 < N / 16; ++c16) {
      v8_t<T> pb;
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[t] = T(s[c16 >> 1][8 * (c16 & 1) + t]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        mma32(ld8<T>(Vt + (db * 32 + a) * C::VS + c16 * 16 + 8 * h2), pb, o[db]);
    }
  }

  // ---- epilogue: normalise and store
  const float l_tot = l_run + xor_lane(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
  T* orow = static_cast<T*>(p.out) + ((size_t(b) * T_ + qa) * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      st4_f32<T>(orow + db * 32 + g4 * 8 + 4 * h2, o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv,
                 o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
  if (p.lse != nullptr && h2 == 0) p.lse[(size_t(b) * Hq + h) * T_ + qa] = (m_run + log2f(l_tot)) * kLn2;
}

template <typename T, int WAVES, int N>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  using C = PrefillCfg<T, WAVES, N>;
  const int n_qt = (a.T + C::M - 1) / C::M;
  const int G = a.Hq / a.Hkv;
  const long long n_groups = (long long)n_qt * a.B * a.Hkv;
  const long long grid = ((n_groups + 7) / 8) * 8 * G;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<T, WAVES, N>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream, a, n_qt,
                     (int)n_groups);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int dtype, const PrefillArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_prefill_t<__bf16, 4, 64>(a, stream);
  return launch_prefill_t<float, 2, 32>(a, stream);
}

}  // namespace relattn
