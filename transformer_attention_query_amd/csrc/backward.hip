// Backward of relative attention for gfx950 (bf16).
//
// Page "SGLang and Miles Add Day-0 Support for Inkling", section "Customized
// Efficient Kernels for Train-Inference Consistency", paragraph "Relative
// attention": the trainer differentiates the attention through the scores
// and through r, P frozen.  With the logit in base-2 units c2*y,
//   y = alpha q.k + [0 <= i-j < E] r_i.P[:, i-j],  c2 = s log2(e),
//   p_ij = exp2(c2 y_ij - lse_i log2(e))           (lse from the forward)
//   dp_ij = dout_i . v_j,  delta_i = dout_i . out_i,  ds_ij = p_ij (dp_ij - delta_i)
//   dq_i = s alpha sum_j ds_ij k_j     dk_j = s alpha sum_i ds_ij q_i
//   dv_j = sum_i p_ij dout_i           dr_i = s sum_{d<E} ds_{i,i-d} P[:, d]
// (the sums over i also run over the query heads of k's and v's group).
//
// Four launches:
//   bwd_delta_kernel   delta_i per (row, head): a dot product of two bf16 rows.
//   bwd_dq_kernel      query-major, like the forward: a wave owns 32 queries
//                      of one head and walks the visible key tiles.  S^T = K Q^T
//                      and the sheared bias as in the forward; dP^T = V dout^T;
//                      dq^T += K^T dS^T (K read transposed from LDS); for band
//                      tiles the wave writes dS^T (bf16) to a private LDS ring
//                      that also holds the previous tile's, and reads it back
//                      along the diagonals (the shear run backwards) as the B
//                      operand of dr^T += P_cols^T G^T, G[i][d] = ds_{i,i-d},
//                      one 32-distance chunk per tile.
//   bwd_dkdv_kernel    key-major: a wave owns 32 keys (their K and V rows stay
//                      in registers as MFMA operands) and walks the query tiles
//                      that see them, for each head of a subset of the group.
//                      S = Q K^T (lane = key), the bias from R^T = P_rows r^T
//                      of the tile's two distance chunks through an LDS shear,
//                      dP = dout V^T, dv^T += dout^T P, dk^T += Q^T dS.
//   bwd_reduce_kernel  when the group's heads are split over workgroups (to
//                      fill the GPU at short lengths): sums the fp32 partials.
#include <climits>

#include "device_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)((__attribute__((address_space(3))) void*)p)));
}

// One bf16 from LDS.  Volatile, because the compiler would otherwise merge
// runs of these into 8-byte reads at 2-byte-aligned addresses, which the LDS
// serves slowly (measured: the whole backward 5 % slower than with single
// reads).
__device__ __forceinline__ __bf16 lds_ld_bf16(const __bf16* p) {
  return *((const volatile __attribute__((address_space(3))) __bf16*)((const __attribute__((address_space(3))) void*)p));
}

// A operand of X^T for a row-major bf16 tile X [rows][STRIDE] in LDS:
// element (i, k-slot t) = X[16*c16 + 8*(t/4) + 4*h + t%4][32*db + i], h =
// lane/32.  That row is the one a 32x32 accumulator register 8*(c16%2) + t of
// the lane holds, so accumulators converted in place are the matching B
// operand.  (Within each 16-lane group G, the transpose read gives lane 4i+e
// element e of the 8 bytes addressed by lane i+4k.)
template <int STRIDE>
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* x, int c16, int db, int lane) {
  const int G = lane >> 4, s = lane & 15, h = G >> 1;
  const __bf16* p0 = x + (16 * c16 + 4 * h + (s >> 2)) * STRIDE + 32 * db + 16 * (G & 1) + 4 * (s & 3);
  const s16x4 a = lds_read_tr(p0);
  const s16x4 b = lds_read_tr(p0 + 8 * STRIDE);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& x, int c16) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = __bf16(x[8 * c16 + t]);
  return r;
}

constexpr int N = 32;          // keys per tile = queries per tile = distances per chunk
constexpr int D = kHeadDim;
constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int XS = D + 24;     // stride of tiles read both by rows and transposed (304-byte rows)
constexpr int RS = D + 8;      // stride of tiles read by rows only (272-byte rows)
constexpr int LS = 2 * N + 4;  // shear buffer row stride (floats)
constexpr int DSS = 104;       // dS^T ring row stride (bf16): three 32-key slots + pad
constexpr int VECS = N * (D / 8) / THREADS;  // 16-byte vectors per thread for a 32 x 128 tile
static_assert(VECS == 2, "tile split");

__device__ __forceinline__ int pos_mod(int k, int m) { return ((k % m) + m) % m; }

// Distance chunk k (distances [32k, 32k+32)) of P_cols, 16-byte vector i of
// this thread, zero outside [0, E) and past d_r.
struct PChunk {
  bf16x8 v[VECS];
  unsigned ok;
  __device__ void fetch(const __bf16* pc, int k, int E, int d_r, int tid) {
    ok = 0;
    const int vpr = d_r / 8;
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      const int d = k * N + (vid >> 4), c8 = vid & 15;
      ok |= unsigned(d >= 0 && d < E && c8 < vpr) << i;
      v[i] = ld8<__bf16>(pc + size_t(min(max(d, 0), max(E - 1, 0))) * d_r + 8 * max(min(c8, vpr - 1), 0));
    }
  }
  template <int STRIDE>
  __device__ void store(__bf16* slot, int tid) const {
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      st8<__bf16>(slot + (vid >> 4) * STRIDE + (vid & 15) * 8, ((ok >> i) & 1u) ? v[i] : zero8<__bf16>());
    }
  }
};

// ---------------------------------------------------------------- delta

__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* out, const __bf16* dout, float* delta, int T,
                                                        int Hq, long long n_rows) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < n_rows) {
    const bf16x8 o = ld8<__bf16>(out + row * D + 8 * l16);
    const bf16x8 g = ld8<__bf16>(dout + row * D + 8 * l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(float(o[e]), float(g[e]), acc);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < n_rows && l16 == 0) {
    const long long bt = row / Hq;
    const int h = int(row % Hq);
    const long long b = bt / T;
    const int t = int(bt % T);
    delta[(b * Hq + h) * T + t] = acc;
  }
}

// ---------------------------------------------------------------- dq, dr

// Workgroup: hpw query heads of one kv head x nqb = WAVES / hpw blocks of 32
// queries (M = 32 nqb consecutive queries).  Wave w: block w / hpw, head
// w % hpw of the subgroup.  The tile's waves read distance chunks
// c0 - 1 .. c0 + nqb - 1 (c0 = (i0 - j0) / 32): a ring of nqb + 1 slots,
// one new chunk per tile.
struct DqLds {
  static constexpr size_t K = size_t(N) * XS * 2;
  static constexpr size_t V = size_t(N) * RS * 2;
  static constexpr size_t P = size_t(WAVES + 1) * N * XS * 2;
  static constexpr size_t R = size_t(WAVES) * N * LS * 4;
  static constexpr size_t G = size_t(WAVES) * N * DSS * 2;
  static constexpr size_t TOTAL = K + V + P + R + G;
  static_assert(TOTAL <= 160 * 1024, "LDS of one workgroup");
};

__global__ __launch_bounds__(THREADS, 1) void bwd_dq_kernel(BackwardArgs p, int n_qt, int n_items, int hpw) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[DqLds::TOTAL];
  __bf16* Ks = reinterpret_cast<__bf16*>(smem);
  __bf16* Vs = reinterpret_cast<__bf16*>(smem + DqLds::K);
  __bf16* Pr = reinterpret_cast<__bf16*>(smem + DqLds::K + DqLds::V);
  float* Rs = reinterpret_cast<float*>(smem + DqLds::K + DqLds::V + DqLds::P);

  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, T = p.T;
  const int d_r = p.d_r, E = p.E, W = p.W;
  const int nqb = WAVES / hpw, M = 32 * nqb, ring = nqb + 1;
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int n_hs = G / hpw;
  const int per_qt = p.B * Hkv * n_hs;
  const int qt = n_qt - 1 - item / per_qt;  // longest rows first
  int rest = item % per_qt;
  const int hs = rest % n_hs;
  rest /= n_hs;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h2 = lane >> 5, a = lane & 31;
  const int qb = w / hpw;
  const int h = kvh * G + hs * hpw + (w % hpw);
  const int i0 = qt * M, qw0 = i0 + 32 * qb, qa = qw0 + a;
  const bool qvalid = qa < T;
  const int qr = qvalid ? qa : T - 1;

  const __bf16* qg = static_cast<const __bf16*>(p.q);
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  // r and P_cols, or any valid address when there is no bias (never read then)
  const __bf16* rg = E > 0 ? static_cast<const __bf16*>(p.r) : qg;
  const __bf16* dog = static_cast<const __bf16*>(p.dout);
  const __bf16* pcg = E > 0 ? static_cast<const __bf16*>(p.pc) : kg;
  const float alpha = p.c1 / p.c2, c2 = p.c2;

  bf16x8 qreg[D / 16], doreg[D / 16], rreg[kMaxDr / 16];
  {
    const size_t row = (size_t(b) * T + qr) * Hq + h;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qreg[kk] = ld8_or_zero<__bf16>(qg + row * D + 8 * h2 + 16 * kk, qvalid);
      doreg[kk] = ld8_or_zero<__bf16>(dog + row * D + 8 * h2 + 16 * kk, qvalid);
    }
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk)
      rreg[kk] = ld8_or_zero<__bf16>(rg + row * d_r + 8 * h2 + 16 * kk, E > 0 && qvalid && kk < d_r / 16);
  }
  const size_t li = (size_t(b) * Hq + h) * T + qr;
  const float lse2 = qvalid ? p.lse[li] * kLog2e : 0.0f;
  const float dl = qvalid ? p.delta[li] : 0.0f;

  f32x16 dq[D / 32], dr[kMaxDr / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = zero16();
#pragma unroll
  for (int i = 0; i < kMaxDr / 32; ++i) dr[i] = zero16();

  const int i_last = min(i0 + M - 1, T - 1);
  const int kt_lo = W > 0 ? max(0, i0 - W + 1) / N : 0;
  const int kt_hi = i_last / N;

  const size_t kv_stride = size_t(Hkv) * D;
  const __bf16* kbase = kg + (size_t(b) * T * Hkv + kvh) * D;
  const __bf16* vbase = vg + (size_t(b) * T * Hkv + kvh) * D;
  bf16x8 kpre[VECS], vpre[VECS];
  auto fetch_kv = [&](int kt) {
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      const int j = min(kt * N + (vid >> 4), T - 1);  // rows past T: clamped, masked later
      const size_t off = size_t(j) * kv_stride + (vid & 15) * 8;
      kpre[i] = ld8<__bf16>(kbase + off);
      vpre[i] = ld8<__bf16>(vbase + off);
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      st8<__bf16>(Ks + (vid >> 4) * XS + (vid & 15) * 8, kpre[i]);
      st8<__bf16>(Vs + (vid >> 4) * RS + (vid & 15) * 8, vpre[i]);
    }
  };
  auto slot = [&](int k) { return Pr + size_t(pos_mod(k, ring)) * N * XS; };
  PChunk pch;

  {
    fetch_kv(kt_lo);
    const int c0 = (i0 - kt_lo * N) / N;
    for (int k = c0 - 1; k <= c0 + nqb - 1; ++k) {
      pch.fetch(pcg, k, E, d_r, tid);
      pch.store<XS>(slot(k), tid);
    }
    store_kv();
  }

  float* rs = Rs + w * N * LS;
  f32x16 rprev = zero16();
  int rlast = INT_MIN;
  // dr runs one distance chunk per tile: chunk c of a tile takes its entries
  // with offset o <= a from this tile's dS and those with o > a from the
  // previous tile's (where it was chunk c-1); glast names the chunk the
  // previous tile's entries still owe.  Row a of the wave's dS^T ring (bf16)
  // has three 32-key slots: a tile of parity p stores its row at slots p and
  // 2 and reads entry o at index 64 - 32p + a - o.  For p = 0 that is slot 2
  // (this tile, o <= a) or slot 1 (the previous, odd tile); for p = 1 slot 1
  // (this tile) or slot 0 (the previous, even tile): one read per entry, no
  // selection.  An odd tile's copy in slot 2 is never read.
  __bf16* grow = reinterpret_cast<__bf16*>(smem + DqLds::K + DqLds::V + DqLds::P + DqLds::R) + (w * N + a) * DSS;
  int glast = INT_MIN;
  auto zero_slot = [&](int off) {  // this lane's 16 entries of one slot
    st8<__bf16>(grow + off + 16 * h2, zero8<__bf16>());
    st8<__bf16>(grow + off + 16 * h2 + 8, zero8<__bf16>());
  };
  auto read_g = [&](int par, bf16x8* g) {
    // k-slot t of step c16 is offset o = 16 c16 + 8(t/4) + 4 h2 + t%4
    const __bf16* rb = grow + (64 - 32 * par) + a - 4 * h2 - 27;
#pragma unroll
    for (int c16 = 0; c16 < 2; ++c16)
#pragma unroll
      for (int t = 0; t < 8; ++t) g[c16][t] = lds_ld_bf16(rb + 27 - (16 * c16 + 8 * (t >> 2) + (t & 3)));
  };
  auto dr_chunk = [&](int k, const bf16x8* g) {
    const __bf16* ps = slot(k);
#pragma unroll
    for (int c16 = 0; c16 < 2; ++c16) {
      bf16x8 pt[kMaxDr / 32];
#pragma unroll
      for (int cb = 0; cb < kMaxDr / 32; ++cb) pt[cb] = frag_tr<XS>(ps, c16, cb, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < kMaxDr / 32; ++cb)
        if (cb < (d_r + 31) / 32) mma32(pt[cb], g[c16], dr[cb]);
    }
  };

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * N;
    const int c0 = (i0 - j0) / N;
    __syncthreads();
    const bool more = kt < kt_hi;
    const int knew = c0 - 2;
    fetch_kv(more ? kt + 1 : kt);
    pch.fetch(pcg, knew, E, d_r, tid);

    const bool wdead = qw0 >= T || j0 > qw0 + 31 || (W > 0 && qw0 - (j0 + N - 1) >= W);
    const bool wband = !wdead && E > 0 && max(0, qw0 - (j0 + N - 1)) < E;
    if (!wband && glast != INT_MIN) {
      // the owed chunk's other entries fall on this tile, which adds none
      // (tiles after a band tile are band tiles or entirely masked): its slot
      // reads as zero.  The P ring still holds the chunk (this tile's chunk c).
      zero_slot(64 - 32 * (kt & 1));
      wave_lds_fence();
      bf16x8 g[2];
      read_g(kt & 1, g);
      dr_chunk(glast, g);
      glast = INT_MIN;
      wave_lds_fence();
    }
    if (!wdead) {
      const bool wmask = (j0 + N - 1 > qw0) || (W > 0 && qw0 + 31 - j0 >= W);
      const int c = c0 + qb;

      // S^T = K Q^T: lane a's column is query a, register v key 8(v/4) + 4 h2 + v%4;
      // dP^T = V dout^T.  One wave per SIMD: every fragment is read from LDS
      // before the first product (the scheduling barrier keeps them there), so
      // each product does not wait for its own read.
      bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) kf[kk] = ld8<__bf16>(Ks + a * XS + 8 * h2 + 16 * kk);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) vf[kk] = ld8<__bf16>(Vs + a * RS + 8 * h2 + 16 * kk);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = zero16(), s2 = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk & 1) mma32(kf[kk], qreg[kk], s2);
        else mma32(kf[kk], qreg[kk], s);
      }
      f32x16 dp = zero16(), dp2 = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk & 1) mma32(vf[kk], doreg[kk], dp2);
        else mma32(vf[kk], doreg[kk], dp);
      }
      if (wband) {
        // R^T of chunks c-1 (new) and c (kept from the previous tile, or made
        // here on the wave's first band tile): R^T = P_rows r^T
        f32x16 racc = zero16();
        {
          const __bf16* pr = slot(c - 1) + a * XS + 8 * h2;
          bf16x8 pf[kMaxDr / 16];
#pragma unroll
          for (int kk = 0; kk < kMaxDr / 16; ++kk) pf[kk] = ld8<__bf16>(pr + 16 * kk);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kk = 0; kk < kMaxDr / 16; ++kk) mma32(pf[kk], rreg[kk], racc);
        }
        if (rlast != c) {
          rprev = zero16();
          const __bf16* pr = slot(c) + a * XS + 8 * h2;
#pragma unroll
          for (int kk = 0; kk < kMaxDr / 16; ++kk) mma32(ld8<__bf16>(pr + 16 * kk), rreg[kk], rprev);
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float* dst = rs + a * LS + 8 * g4 + 4 * h2;
          f32x4 x0, x1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[e] = racc[4 * g4 + e];
            x1[e] = rprev[4 * g4 + e];
          }
          *reinterpret_cast<f32x4*>(dst) = x0;
          *reinterpret_cast<f32x4*>(dst + 32) = x1;
        }
        rprev = racc;
        rlast = c - 1;
        wave_lds_fence();
        // key b of query a is at distance 32c + a - b: column 32 + a - b
        const float* src = rs + a * LS + 32 + a - 4 * h2;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = fmaf(s[v] + s2[v], alpha, src[-(8 * (v >> 2) + (v & 3))]);
        wave_lds_fence();
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (s[v] + s2[v]) * alpha;
      }
      if (wmask) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int dd = qa - (j0 + 8 * (v >> 2) + 4 * h2 + (v & 3));
          if (dd < 0 || (W > 0 && dd >= W)) s[v] = -INFINITY;
        }
      }
      // dS^T = P^T (dP^T - delta)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = fast_exp2(fmaf(s[v], c2, -lse2)) * (dp[v] + dp2[v] - dl);
      // dq^T += K^T dS^T
      bf16x8 sb[2];
#pragma unroll
      for (int c16 = 0; c16 < 2; ++c16) {
        bf16x8 kt_f[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) kt_f[db] = frag_tr<XS>(Ks, c16, db, lane);
        __builtin_amdgcn_sched_barrier(0);
        sb[c16] = to_bf16x8(s, c16);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) mma32(kt_f[db], sb[c16], dq[db]);
      }
      if (wband) {
        // dS^T (the bf16 operands of the dq product) to row a of the ring:
        // key 8 g4 + 4 h2 + e is element 4 g4 + e of the lane's sixteen
        const int par = kt & 1;
        if (glast != c) zero_slot(32 * (1 - par));  // no previous tile owes this chunk
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = sb[g4 >> 1][4 * (g4 & 1) + e];
          *reinterpret_cast<bf16x4*>(grow + 32 * par + 8 * g4 + 4 * h2) = x;
          *reinterpret_cast<bf16x4*>(grow + 64 + 8 * g4 + 4 * h2) = x;
        }
        wave_lds_fence();
        // dr^T += P_cols^T G^T, G[a][32k + o] = dS[a][key a + 32(c - k) - o]
        bf16x8 g[2];
        read_g(par, g);
        dr_chunk(c, g);
        glast = c - 1;
        wave_lds_fence();
      }
    }

    __syncthreads();
    if (more) {
      store_kv();
      pch.store<XS>(slot(knew), tid);
    }
  }

  if (glast != INT_MIN) {  // the last owed chunk (no further tile adds to it)
    zero_slot(64 - 32 * ((kt_hi + 1) & 1));
    wave_lds_fence();
    bf16x8 g[2];
    read_g((kt_hi + 1) & 1, g);
    dr_chunk(glast, g);
  }

  // ---- epilogue: dq = s alpha dq^T^T, dr = s dr^T^T through a per-wave LDS
  // staging tile, written back as whole rows
  __syncthreads();
  constexpr int OS = D + 8;
  __bf16* ot = reinterpret_cast<__bf16*>(smem) + size_t(w) * 32 * OS;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  auto emit = [&](auto& acc, int nblk, float scale, __bf16* dst, int row_len) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
      if (db < nblk)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          st4_f32<__bf16>(ot + a * OS + db * 32 + g4 * 8 + 4 * h2, acc[db][4 * g4] * scale,
                          acc[db][4 * g4 + 1] * scale, acc[db][4 * g4 + 2] * scale, acc[db][4 * g4 + 3] * scale);
    wave_lds_fence();
    const int vpr = row_len / 8;
    for (int i = lane; i < 32 * vpr; i += 64) {
      const int row = i / vpr, cv = i % vpr;
      const int q = qw0 + row;
      if (q < T)
        *reinterpret_cast<u32x4*>(dst + ((size_t(b) * T + q) * Hq + h) * row_len + cv * 8) =
            *reinterpret_cast<const u32x4*>(ot + row * OS + cv * 8);
    }
    wave_lds_fence();
  };
  emit(dq, D / 32, p.sa, static_cast<__bf16*>(p.dq), D);
  if (p.dr != nullptr && d_r > 0) emit(dr, (d_r + 31) / 32, p.s, static_cast<__bf16*>(p.dr), d_r);
}

// ---------------------------------------------------------------- dk, dv

// Workgroup: WAVES waves x 32 keys = one 128-key block of one kv head, for
// the heads hs*hps .. hs*hps + hps - 1 of its group.  Steps run over the
// query tiles that see the block (outer) and the heads (inner); a step stages
// the tile's q, dout, r rows, lse and delta of one head in LDS.  The waves'
// distance chunks at query tile it are cb-4 .. cb (cb = it - j0/32): a ring
// of 8 slots, one new chunk per query tile.
struct DkvLds {
  static constexpr size_t Q = size_t(N) * XS * 2;
  static constexpr size_t DO = size_t(N) * XS * 2;
  static constexpr size_t RR = size_t(N) * RS * 2;
  static constexpr size_t LD = 2 * N * 4;
  static constexpr int RING = 8;
  static constexpr size_t P = size_t(RING) * N * RS * 2;
  static constexpr size_t R = size_t(WAVES) * N * LS * 4;
  static constexpr size_t TOTAL = Q + DO + RR + LD + P + R;
  static_assert(TOTAL <= 160 * 1024, "LDS of one workgroup");
};

__global__ __launch_bounds__(THREADS, 1) void bwd_dkdv_kernel(BackwardArgs p, int n_kb, int n_items) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[DkvLds::TOTAL];
  __bf16* Qs = reinterpret_cast<__bf16*>(smem);
  __bf16* Ds = reinterpret_cast<__bf16*>(smem + DkvLds::Q);
  __bf16* Rr = reinterpret_cast<__bf16*>(smem + DkvLds::Q + DkvLds::DO);
  float* Ls = reinterpret_cast<float*>(smem + DkvLds::Q + DkvLds::DO + DkvLds::RR);  // lse2 [32], delta [32]
  __bf16* Pr = reinterpret_cast<__bf16*>(smem + DkvLds::Q + DkvLds::DO + DkvLds::RR + DkvLds::LD);
  float* Rs = reinterpret_cast<float*>(smem + DkvLds::Q + DkvLds::DO + DkvLds::RR + DkvLds::LD + DkvLds::P);

  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv, T = p.T;
  const int d_r = p.d_r, E = p.E, W = p.W;
  const int n_split = p.n_split, hps = G / n_split;
  const int item = blockIdx.x;
  if (item >= n_items) return;
  // Under the causal mask the blocks run longest first (block 0 sees every
  // query).  In a sliding-window layer every block has the same work, and
  // consecutive blocks of one (batch, kv head, split) go to one XCD
  // (workgroup i runs on XCD i % 8), so the query tiles they share meet in
  // that XCD's L2.
  const int per_kb = p.B * Hkv * n_split;
  int kb, rest;
  if (W > 0 && n_items % 8 == 0) {
    const int lin = (item % 8) * (n_items / 8) + item / 8;
    kb = lin % n_kb;
    rest = lin / n_kb;
  } else {
    kb = item / per_kb;
    rest = item % per_kb;
  }
  const int hs = rest % n_split;
  rest /= n_split;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h2 = lane >> 5, a = lane & 31;
  const int j0 = kb * (N * WAVES), j0w = j0 + N * w;
  const int key = j0w + a;
  const bool kvalid = key < T;

  const __bf16* qg = static_cast<const __bf16*>(p.q);
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  const __bf16* rg = E > 0 ? static_cast<const __bf16*>(p.r) : qg;
  const __bf16* dog = static_cast<const __bf16*>(p.dout);
  const __bf16* pcg = E > 0 ? static_cast<const __bf16*>(p.pc) : kg;
  const float alpha = p.c1 / p.c2, c2 = p.c2;

  // this lane's key and value rows as B operands (column = key a)
  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const size_t row = (size_t(b) * T + (kvalid ? key : T - 1)) * Hkv + kvh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kreg[kk] = ld8_or_zero<__bf16>(kg + row * D + 8 * h2 + 16 * kk, kvalid);
      vreg[kk] = ld8_or_zero<__bf16>(vg + row * D + 8 * h2 + 16 * kk, kvalid);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  const int it_lo = j0 / N;
  const int q_end = W > 0 ? min(T, j0 + N * WAVES - 1 + W) : T;  // queries [j0, q_end) see the block
  const int it_hi = (q_end - 1) / N;
  const int h_first = kvh * G + hs * hps;

  // staged step (query tile it, head h): q, dout and r rows, lse2 and delta
  bf16x8 qpre[VECS], dpre[VECS], rpre[VECS];
  float lpre = 0.0f;
  // Every load is issued unconditionally from a clamped address inside its
  // tensor (rows past T read row T-1, columns past d_r the row's last piece,
  // r without bias reads q); rows past T and columns past d_r are zeroed when
  // stored, so no load sits behind a branch.
  unsigned pre_ok = 0;  // bit i: vector i's row is a query; bit 8 + i: its r piece is needed
  const float* lsrc = tid < N ? p.lse : p.delta;
  auto fetch_step = [&](int it, int h) {
    pre_ok = 0;
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      const int qi = it * N + (vid >> 4), c8 = vid & 15;
      const bool ok = qi < T;
      pre_ok |= (unsigned(ok) << i) | (unsigned(ok && E > 0 && c8 < d_r / 8) << (8 + i));
      const size_t row = (size_t(b) * T + min(qi, T - 1)) * Hq + h;
      qpre[i] = ld8<__bf16>(qg + row * D + 8 * c8);
      dpre[i] = ld8<__bf16>(dog + row * D + 8 * c8);
      rpre[i] = ld8<__bf16>(rg + (E > 0 ? row * d_r + 8 * min(c8, max(d_r / 8 - 1, 0)) : row * D + 8 * c8));
    }
    if (tid < 2 * N) {
      const int qi = it * N + (tid & (N - 1));
      lpre = lsrc[(size_t(b) * Hq + h) * T + min(qi, T - 1)];
      pre_ok |= unsigned(qi < T) << 16;
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      const int vid = tid + i * THREADS;
      const int row = vid >> 4, c8 = vid & 15;
      const bool ok = (pre_ok >> i) & 1u, rok = (pre_ok >> (8 + i)) & 1u;
      st8<__bf16>(Qs + row * XS + c8 * 8, ok ? qpre[i] : zero8<__bf16>());
      st8<__bf16>(Ds + row * XS + c8 * 8, ok ? dpre[i] : zero8<__bf16>());
      st8<__bf16>(Rr + row * RS + c8 * 8, rok ? rpre[i] : zero8<__bf16>());
    }
    if (tid < 2 * N) Ls[tid] = ((pre_ok >> 16) & 1u) ? (tid < N ? lpre * kLog2e : lpre) : 0.0f;
  };
  auto slot = [&](int k) { return Pr + size_t(k & (DkvLds::RING - 1)) * N * RS; };
  PChunk pch;

  auto fill_ring = [&](int it) {  // the WAVES + 1 chunks of query tile it
    const int cb = it - j0 / N;
    for (int k = cb - WAVES; k <= cb; ++k) {
      pch.fetch(pcg, k, E, d_r, tid);
      pch.store<RS>(slot(k), tid);
    }
  };

  // Order of the query tiles.  In a sliding-window layer a full block sees
  // n_rot tiles; step sg takes the block's tile congruent to sg modulo n_rot,
  // so at any step all the blocks that share a tile take it together (and
  // its rows are read from L2 once for them).  A block cut short by the end of
  // the sequence skips the steps whose tile lies past it.  Causal: ascending.
  const int n_rot = W > 0 ? (N * WAVES - 2 + W) / N + 1 : it_hi - it_lo + 1;
  auto tile_at = [&](int sg) { return W > 0 ? it_lo + pos_mod(sg - it_lo, n_rot) : it_lo + sg; };
  auto next_valid = [&](int sg) {
    while (sg < n_rot && tile_at(sg) > it_hi) ++sg;
    return sg;
  };
  int sg = next_valid(0);
  int it = tile_at(sg);
  fetch_step(it, h_first);
  fill_ring(it);
  store_step();

  float* rs = Rs + w * N * LS;
  while (sg < n_rot) {
    const int i0 = it * N;
    const int sg_next = next_valid(sg + 1);
    const int it_next = sg_next < n_rot ? tile_at(sg_next) : -1;
    const bool adjacent = it_next == it + 1;  // the ring then takes one new chunk
    for (int hh = 0; hh < hps; ++hh) {
      __syncthreads();
      const bool last_h = hh + 1 == hps;
      const bool more = !(last_h && it_next < 0);
      if (more) fetch_step(last_h ? it_next : it, h_first + (last_h ? 0 : hh + 1));
      const int knew = it_next - j0 / N;  // chunk the next query tile adds
      if (last_h && more && adjacent) pch.fetch(pcg, knew, E, d_r, tid);

      const bool wdead = j0w >= T || i0 + 31 < j0w || (W > 0 && i0 - (j0w + N - 1) >= W);
      if (!wdead) {
        const bool wband = E > 0 && max(0, i0 - (j0w + N - 1)) < E;
        const bool wmask = (j0w + N - 1 > i0) || (W > 0 && i0 + 31 - j0w >= W) || i0 + 31 >= T;
        // S = Q K^T: lane a's column is key a, register v query 8(v/4) + 4 h2 + v%4;
        // dP = dout V^T.  One wave per SIMD: every fragment is read from LDS
        // before the first product (the scheduling barrier keeps them there),
        // so each product does not wait for its own read.
        bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qf[kk] = ld8<__bf16>(Qs + a * XS + 8 * h2 + 16 * kk);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) df[kk] = ld8<__bf16>(Ds + a * XS + 8 * h2 + 16 * kk);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s = zero16(), s2 = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk & 1) mma32(qf[kk], kreg[kk], s2);
          else mma32(qf[kk], kreg[kk], s);
        }
        f32x16 dp = zero16(), dp2 = zero16();
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk & 1) mma32(df[kk], vreg[kk], dp2);
          else mma32(df[kk], vreg[kk], dp);
        }
        if (wband) {
          // R^T of the wave's chunks cw-1 and cw (query a of the tile and key b
          // of the wave are 32 cw + a - b apart): lane a's column is query a
          const int cw = (i0 - j0w) / N;
          f32x16 r0 = zero16(), r1 = zero16();
          const __bf16* p0 = slot(cw - 1) + a * RS + 8 * h2;
          const __bf16* p1 = slot(cw) + a * RS + 8 * h2;
          const __bf16* rt = Rr + a * RS + 8 * h2;
#pragma unroll
          for (int half = 0; half < kMaxDr / 64; ++half) {
            // four fragments of each operand at a time (all eight would spill)
            bf16x8 rf[4], f0[4], f1[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
              const int kk = 4 * half + k4;
              rf[k4] = ld8<__bf16>(rt + 16 * kk);
              f0[k4] = ld8<__bf16>(p0 + 16 * kk);
              f1[k4] = ld8<__bf16>(p1 + 16 * kk);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
              mma32(f0[k4], rf[k4], r0);
              mma32(f1[k4], rf[k4], r1);
            }
          }
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float* dst = rs + a * LS + 8 * g4 + 4 * h2;
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x0[e] = r0[4 * g4 + e];
              x1[e] = r1[4 * g4 + e];
            }
            *reinterpret_cast<f32x4*>(dst) = x0;
            *reinterpret_cast<f32x4*>(dst + 32) = x1;
          }
          wave_lds_fence();
          // query a' = 8(v/4) + 4 h2 + v%4 and key a: row a', column 32 + a' - a
          const float* src = rs + 32 - a;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qv = 8 * (v >> 2) + 4 * h2 + (v & 3);
            s[v] = fmaf(s[v] + s2[v], alpha, src[qv * (LS + 1)]);
          }
          wave_lds_fence();
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = (s[v] + s2[v]) * alpha;
        }
        if (wmask) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qi = i0 + 8 * (v >> 2) + 4 * h2 + (v & 3);
            const int dd = qi - key;
            if (dd < 0 || (W > 0 && dd >= W) || qi >= T) s[v] = -INFINITY;
          }
        }
        // P and dS = P (dP - delta), per query row
        f32x16 pp;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + 8 * g4 + 4 * h2);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ls + N + 8 * g4 + 4 * h2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g4 + e;
            pp[v] = fast_exp2(fmaf(s[v], c2, -l4[e]));
            s[v] = pp[v] * (dp[v] + dp2[v] - d4[e]);
          }
        }
        // dv^T += dout^T P, dk^T += Q^T dS
#pragma unroll
        for (int c16 = 0; c16 < 2; ++c16) {
          bf16x8 fd[D / 32], fq[D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            fd[db] = frag_tr<XS>(Ds, c16, db, lane);
            fq[db] = frag_tr<XS>(Qs, c16, db, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 pb = to_bf16x8(pp, c16);
          const bf16x8 sb = to_bf16x8(s, c16);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            mma32(fd[db], pb, dv[db]);
            mma32(fq[db], sb, dk[db]);
          }
        }
      }

      __syncthreads();
      if (more) store_step();
      if (last_h && more) {
        if (adjacent) pch.store<RS>(slot(knew), tid);
        else fill_ring(it_next);
      }
    }
    sg = sg_next;
    it = it_next;
  }

  // ---- epilogue: rows of dk (scaled by s alpha) and dv, bf16 or fp32 partials
  __syncthreads();
  constexpr int OS = D + 4;
  float* ot = reinterpret_cast<float*>(smem) + size_t(w) * 32 * OS;
  auto emit = [&](auto& acc, float scale, int which) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g4 + e] * scale;
        *reinterpret_cast<f32x4*>(ot + a * OS + db * 32 + g4 * 8 + 4 * h2) = x;
      }
    wave_lds_fence();
    for (int i = lane; i < 32 * (D / 4); i += 64) {
      const int row = i / (D / 4), c4 = i % (D / 4);
      const int j = j0w + row;
      if (j >= T) continue;
      const f32x4 x = *reinterpret_cast<const f32x4*>(ot + row * OS + 4 * c4);
      const size_t off = ((size_t(b) * T + j) * Hkv + kvh) * D + 4 * c4;
      if (n_split == 1) {
        st4_f32<__bf16>(static_cast<__bf16*>(which ? p.dv : p.dk) + off, x[0], x[1], x[2], x[3]);
      } else {
        const size_t plane = size_t(p.B) * T * Hkv * D;
        *reinterpret_cast<f32x4*>(p.part + (size_t(hs) * 2 + which) * plane + off) = x;
      }
    }
    wave_lds_fence();
  };
  emit(dk, p.sa, 0);
  emit(dv, 1.0f, 1);
}

// ---------------------------------------------------------------- head-split sum

__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* part, __bf16* dk, __bf16* dv, size_t plane,
                                                         int n_split) {
  const size_t i = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= 2 * plane) return;
  const int which = i >= plane;
  const size_t off = i - (which ? plane : 0);
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + which * plane + off);
  for (int sp = 1; sp < n_split; ++sp) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(part + (size_t(sp) * 2 + which) * plane + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += x[e];
  }
  st4_f32<__bf16>((which ? dv : dk) + off, acc[0], acc[1], acc[2], acc[3]);
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.T * a.Hq;
  bwd_delta_kernel<<<dim3(unsigned((rows + 15) / 16)), dim3(256), 0, stream>>>(
      static_cast<const __bf16*>(a.out), static_cast<const __bf16*>(a.dout), a.delta, a.T, a.Hq, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // dq / dr: heads per workgroup = largest power of two <= WAVES dividing G
  const int G = a.Hq / a.Hkv;
  int hpw = 1;
  while (hpw * 2 <= WAVES && G % (hpw * 2) == 0) hpw *= 2;
  const int M = 32 * (WAVES / hpw);
  const int n_qt = (a.T + M - 1) / M;
  const int n_items = n_qt * a.B * a.Hkv * (G / hpw);
  bwd_dq_kernel<<<dim3(unsigned(n_items)), dim3(THREADS), 0, stream>>>(a, n_qt, n_items, hpw);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_kb = (a.T + N * WAVES - 1) / (N * WAVES);
  const int n_kv = n_kb * a.B * a.Hkv * a.n_split;
  bwd_dkdv_kernel<<<dim3(unsigned(n_kv)), dim3(THREADS), 0, stream>>>(a, n_kb, n_kv);
  e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;

  const size_t plane = size_t(a.B) * a.T * a.Hkv * D;
  bwd_reduce_kernel<<<dim3(unsigned((2 * plane / 4 + 255) / 256)), dim3(256), 0, stream>>>(
      a.part, static_cast<__bf16*>(a.dk), static_cast<__bf16*>(a.dv), plane, a.n_split);
  return hipGetLastError();
}

}  // namespace relattn
