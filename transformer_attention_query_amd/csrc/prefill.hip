// Relative-attention prefill for gfx950.
//
// Computes, for every query i of a sequence and query head h (page "SGLang
// and Miles Add Day-0 Support for Inkling", section "Attention with Relative
// Positional Embedding", eqs. for rel_logits and l(i,j,h)):
//   l(i,j) = s*alpha*q_i.k_j + [0 <= i-j < E] * s * r_i.P[:, i-j]
// under the causal / sliding-window mask, then the softmax over j and the
// weighted sum of v_j, in one pass (online softmax with the bias added before
// the running max, as the FA4 fork does -- section "Relative Logits
// Optimization", Figure 3).
//
// Work decomposition
//   * One workgroup = WAVES waves = M = 32*WAVES consecutive queries of one
//     (batch, query head); it walks the key tiles of N keys that the mask
//     leaves visible (tiles entirely in the future or entirely outside the
//     window are never touched).
//   * Scores are computed transposed, S^T = K Q^T, so lane l of a wave owns
//     query l%32 and the 32x32 MFMA accumulators run over keys: the row max
//     and row sum are in-lane reductions plus one exchange with lane l^32, and
//     the output accumulator O^T = V^T P^T needs no cross-lane traffic.
//   * K tiles are staged in LDS row-major.  bf16 V tiles are staged row-major
//     too and read as MFMA fragments with the gfx950 transpose read
//     (ds_read_b64_tr_b16); fp32 V tiles are stored transposed.
//   * Relative bias ("sheared bias" of section "Relative Logits
//     Optimization": bias(i,j) = rel_logits(i, i-j)) is formed per wave.  The
//     wave's queries start Dw = 32c keys after the tile's first key, so query
//     a and key b are 32c + a - b apart: distance chunks c-1 (a < b) and c
//     (a >= b), 32 distances each.  Chunk c was made on the previous key tile;
//     only chunk c-1 is new: R^T = P_rows r^T over its 32 distances, one MFMA
//     chain the length of the QK chain.  R goes to a wave-private LDS buffer
//     [query][distance] (two chunk slots, even chunks also in a third so the
//     pair is always contiguous) and is read back along the shear: a lane
//     only reads its own query's row.  Distances outside [0, E) read zero P
//     rows, so the rel_extent cut needs no per-score test.
//   * P rows live in a ring of N-row chunks in LDS.  A tile's window of
//     distances [D0 - N, D0 + M) is M/N + 1 consecutive chunks (D0 = first
//     query minus first key); moving one tile right slides the window down by
//     one chunk, so each tile fetches a single new chunk, into a slot the
//     current window does not use.
//   * The next tile's K, V and P chunk are fetched into registers while the
//     current tile computes and are written to LDS between two barriers.
//     (bf16 with eight or more query heads per kv head takes
//     prefill_dma_kernel below instead: LDS DMA into double-buffered tiles,
//     one barrier per tile, and a tile loop software-pipelined per wave.)
//   * Softmax works in units of c2 = s*log2(e): y = S*(c1/c2) + R, so the bias
//     rows need no scaling, and p = exp2(c2*y - c2*m).  O is rescaled only
//     when a row maximum grows by more than 2^8 (exact either way: O and l
//     share the stale maximum).
#include <climits>

#include "device_common.hpp"
#include "mx_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;
// Largest sum of one lane's 16 exponentials (taken against the running
// maximum) that the DMA kernel's tile loop accepts without raising the
// maximum: 2^12, so every p stays at most 4096.
constexpr float kPsumLimit = 4096.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned char u8;

// MXFP8 K tile of the extend form over MXFP8 caches: E4M3 codes [N keys][KCS
// bytes] and the E8M0 scales [N keys][4], in the K tile's LDS.
constexpr int kMxKcs = kHeadDim + 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)((__attribute__((address_space(3))) void*)p)));
}

// V tile staging and PV A-operand fragments.  The PV MFMA's k-slot 8*h + t
// (h = lane/32) holds key 16*c16 + 8*(t/4) + 4*h + t%4 of 16-key chunk c16:
// the key the S^T accumulator register 8*(c16%2) + t of that lane holds.
template <typename T, int N> struct PreV;

template <int N> struct PreV<__bf16, N> {
  // Row-major [N keys][160]: 320-byte rows put the 4 rows x 64 bytes a
  // half-wave transpose read touches in distinct bank groups.
  static constexpr int ROW = 160;
  static constexpr size_t BYTES = size_t(N) * ROW * sizeof(__bf16);
  __device__ static void store(__bf16* vs, int row, int c8, const bf16x8& x) { st8<__bf16>(vs + row * ROW + c8 * 8, x); }
  // Within each 16-lane group G, result lane 4i+e element k is element e of
  // the 8 bytes addressed by lane i+4k: lane (G, s) addresses key row
  // 16*c16 + 4*h + s/4 (then +8) at columns 32*db + 16*(G%2) + 4*(s%4).
  __device__ static bf16x8 frag(const __bf16* vs, int c16, int db, int lane) {
    const int G = lane >> 4, s = lane & 15, h = G >> 1;
    const __bf16* p0 = vs + (16 * c16 + 4 * h + (s >> 2)) * ROW + 32 * db + 16 * (G & 1) + 4 * (s & 3);
    const s16x4 a = lds_read_tr(p0);
    const s16x4 b = lds_read_tr(p0 + 8 * ROW);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

template <int N> struct PreV<float, N> {
  // Transposed [128 d][N + 4]; key `row` sits at the slot where the middle two
  // groups of four of its 16-key chunk are swapped.
  static constexpr int VS = N + 4;
  static constexpr size_t BYTES = size_t(kHeadDim) * VS * sizeof(float);
  __device__ static int pos(int row) {
    const int k16 = row & 15;
    return (row & ~15) + ((k16 >> 2) & 1) * 8 + (k16 >> 3) * 4 + (k16 & 3);
  }
  __device__ static void store(float* vs, int row, int c8, const f32x8& x) {
    const int p = pos(row);
#pragma unroll
    for (int e = 0; e < 8; ++e) vs[(c8 * 8 + e) * VS + p] = x[e];
  }
  __device__ static f32x8 frag(const float* vs, int c16, int db, int lane) {
    const int a = lane & 31, h = lane >> 5;
    return ld8<float>(vs + (32 * db + a) * VS + 16 * c16 + 8 * h);
  }
};

template <typename T, int WAVES>
struct PrefillCfg {
  static constexpr int N = 32;                // keys per tile = distances per chunk
  static constexpr int M = 32 * WAVES;        // queries per workgroup
  static constexpr int PAD = 16 / sizeof(T);  // 16 bytes of padding per K / P row
  static constexpr int KS = kHeadDim + PAD;   // K tile row stride (elements)
  static constexpr int PS = kMaxDr + PAD;     // P ring row stride (elements)
  // A tile reads one new chunk per wave, WAVES consecutive chunks; the next
  // tile's new chunk replaces the highest of them after the end-of-tile
  // barrier, so the ring is exactly WAVES slots.
  static constexpr int RING = WAVES;
  static constexpr int LS = 2 * N + 4;        // R buffer row stride (floats): 64 columns + 4
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KV_VECS = N * (kHeadDim / 8) / THREADS;  // 8-element vectors per thread per tile
  static constexpr int P_VECS = N * (kMaxDr / 8) / THREADS;     // per thread per P chunk (d_r = 128)
  static constexpr size_t LDS_K = size_t(N) * KS * sizeof(T);
  static constexpr size_t LDS_V = PreV<T, N>::BYTES;
  static constexpr size_t LDS_P = size_t(RING) * N * PS * sizeof(T);
  static constexpr size_t LDS_R = size_t(WAVES) * 32 * LS * sizeof(float);
  static constexpr size_t LDS_TOTAL = LDS_K + LDS_V + LDS_P + LDS_R;
  static_assert((RING & (RING - 1)) == 0, "ring slots are chunk & (RING-1)");
  static_assert(KV_VECS >= 1 && KV_VECS * THREADS == N * (kHeadDim / 8), "tile must split evenly over threads");
  static_assert(P_VECS >= 1 && P_VECS * THREADS == N * (kMaxDr / 8), "chunk must split evenly over threads");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// EXT: the extend form (new rows of packed sequences over their KV caches,
// contiguous or paged; see rel_attn_extend).  Positions are global: query
// row t of sequence b sits at kv_len[b] - n_b + t, and query tiles are
// aligned to multiples of M positions, so the chunk arithmetic is unchanged.
// MX (bf16, EXT): the caches hold MXFP8 (E4M3 codes, one E8M0 scale per 32
// values of D; page "SGLang and Miles Add Day-0 Support for Inkling",
// section "Relative Logits Optimization", paragraph "MXFP8 Support").  The
// query is quantised to MXFP8 the same way and the scores come from the
// MX-scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, two per 32x32
// tile); V is dequantised to bf16 (exactly) when its tile is staged.
template <typename T, int WAVES, bool EXT, bool MX = false>
__global__ __launch_bounds__(WAVES * 64, 1) void prefill_kernel(PrefillArgs p, int n_qt, int n_items, int hpw) {
  static_assert(!MX || (EXT && sizeof(T) == 2), "MXFP8 caches: the bf16 extend form");
  using C = PrefillCfg<T, WAVES>;
  using VS = PreV<T, C::N>;
  constexpr int N = C::N;
  constexpr int D = kHeadDim;

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_TOTAL];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = reinterpret_cast<T*>(smem + C::LDS_K);
  T* Pr = reinterpret_cast<T*>(smem + C::LDS_K + C::LDS_V);
  float* Rs = reinterpret_cast<float*>(smem + C::LDS_K + C::LDS_V + C::LDS_P);

  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const int d_r = p.d_r, E = p.E, W = p.W;

  // ---- workgroup -> (q-tile, batch, kv head, head subgroup); wave -> (query
  // block, query head).  The waves of a workgroup are hpw query heads of one
  // kv head (GQA packing) times nqb = WAVES/hpw blocks of 32 queries: with
  // hpw = WAVES every wave sees the same keys, the same masks and the same
  // distance chunks, so no wave idles at a barrier and one P chunk serves
  // all.  Work items are ordered longest-first (late q-tiles see the most
  // keys under the causal mask); item i and i+8 share an XCD and are nearby
  // q-tiles of one kv head, so their K/V tiles meet in that XCD's L2.
  const int nqb = WAVES / hpw;
  const int M = 32 * nqb;
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int n_hs = G / hpw;
  const int per_qt = p.B * Hkv * n_hs;
  const int qt = n_qt - 1 - item / per_qt;
  int rest = item % per_qt;
  const int hs = rest % n_hs;
  rest /= n_hs;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;  // half-wave
  const int a = lane & 31;   // this lane's query within the wave
  const int qb = w / hpw;    // query block of this wave
  const int h = kvh * G + hs * hpw + (w % hpw);

  // T_: keys (and positions) of this sequence; [pos0, T_) are its query
  // positions, packed from row row0 of q, r and out
  int T_ = p.T, pos0 = 0, row0 = 0;
  float c1 = p.c1, c2 = p.c2;
  int qt_abs = qt;
  if constexpr (EXT) {
    const int cap = p.btab != nullptr ? p.max_pages * p.page_size : p.cap;
    T_ = max(0, min(p.kv_len[b], cap));
    row0 = min(max(p.q_start[b], 0), p.total_q);
    const int n = max(0, min(min(p.q_start[b + 1] - p.q_start[b], min(T_, p.max_q)), p.total_q - row0));
    pos0 = T_ - n;
    qt_abs = pos0 / M + qt;
    if (n == 0 || qt_abs * M >= T_) return;
    if (p.log_scale) {  // s = max(1, ln(kv_len) / ln(4096)), one per sequence
      const float sc = fmaxf(1.0f, logf(float(T_)) * (1.0f / 8.317766166719343f));
      c2 = sc * 1.4426950408889634f;
      c1 = c2 * p.alpha;
    }
  }
  const int i0 = qt_abs * M;
  const int qw0 = i0 + 32 * qb;
  const int qa = qw0 + a;
  const bool qvalid = qa >= pos0 && qa < T_;
  // packed row of query position x of this sequence (plain prefill: b*T + x)
  auto qrow_of = [&](int x) -> size_t {
    if constexpr (EXT) return size_t(row0 + x - pos0);
    else return size_t(b) * T_ + x;
  };

  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  const T* rg = static_cast<const T*>(p.r);
  // P_cols, or any valid address when there is no bias (its loads are then discarded)
  const T* pcg = E > 0 ? static_cast<const T*>(p.pc) : kg;

  // softmax constants in units of c2 (c2 = s*log2(e) > 0)
  const float qk_scale = c1 / c2;
  const float lazy = kLazyRescaleLog2 / c2;

  // ---- this lane's query and relative feature, as MFMA B operands
  v8_t<T> qreg[D / 16];
  i32x8 qx[2];             // MX: the query's E4M3 bytes for score MFMA m = 0, 1
  int qsc[2] = {127, 127};  // MX: E8M0 scale this lane supplies to MFMA m
  if constexpr (!MX) {
    const T* qrow = qg + (qrow_of(qvalid ? qa : pos0) * Hq + h) * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = ld8_or_zero<T>(qrow + kk * 16, qvalid);
  } else {
    // Operand layout of the 32x32x64 scaled MFMA (checked on the device):
    // lane (h2, a) holds, for row/column a, bytes k = 16*h2 + t (t < 16) and
    // 32 + 16*h2 + (t - 16) (t >= 16) of the instruction's 64, and supplies
    // the scale of row/column a for its 32-value block h2.  Score MFMA m
    // covers d = 64m .. 64m+63, so this lane holds half h2 of each of the
    // four d-blocks of its query; each block's maximum joins the two halves
    // (lanes l and l ^ 32).
    const T* qrow = qg + (qrow_of(qvalid ? qa : pos0) * Hq + h) * D + 16 * h2;
    float qv[4][16];  // [block][t]: d = 32*block + 16*h2 + t
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const v8_t<T> x0 = ld8_or_zero<T>(qrow + 32 * blk, qvalid);
      const v8_t<T> x1 = ld8_or_zero<T>(qrow + 32 * blk + 8, qvalid);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[blk][e] = float(x0[e]);
        qv[blk][8 + e] = float(x1[e]);
      }
    }
    int sh[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      float amax = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(qv[blk][t]));
      sh[blk] = mx_shared_exp(pair_max32(amax));
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const float* lo = &qv[2 * m][4 * w4];
        const float* hi = &qv[2 * m + 1][4 * w4];
        qx[m][w4] = int(e4m3_pack4(lo[0], lo[1], lo[2], lo[3], sh[2 * m]));
        qx[m][4 + w4] = int(e4m3_pack4(hi[0], hi[1], hi[2], hi[3], sh[2 * m + 1]));
      }
      // arithmetic pick (an indexed pick would put sh[] in scratch memory)
      qsc[m] = 127 + sh[2 * m] + h2 * (sh[2 * m + 1] - sh[2 * m]);
    }
  }
  v8_t<T> rreg[kMaxDr / 16];  // zero past d_r
  {
    const int nkr = d_r / 16;
    const T* rrow = rg + (qrow_of(qvalid ? qa : pos0) * Hq + h) * d_r + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) rreg[kk] = ld8_or_zero<T>(rrow + kk * 16, E > 0 && qvalid && kk < nkr);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();
  // running max (units of c2), finite so exp2 of a masked score is exactly 0
  float m_run = -1e30f;
  float l_run = 0.0f;

  // ---- visible key tiles of this q-tile
  const int i_last = min(i0 + M - 1, T_ - 1);
  int kt_lo = 0;
  if (W > 0) kt_lo = max(0, i0 - W + 1) / N;
  const int kt_hi = i_last / N;

  // ---- K/V tile and P chunk prefetch through registers
  // Key j of this sequence: row b*cap + j of a contiguous cache (b*T + j in
  // plain prefill), or slot j % page_size of page btab[b][j / page_size] of
  // a paged one (page_size a multiple of N, so a tile lies in one page; page
  // ids are clamped to the pool).
  const size_t seq_rows = EXT ? size_t(p.cap) : size_t(T_);
  v8_t<T> kpre[C::KV_VECS], vpre[C::KV_VECS];
  // MX: codes of the same 8 values (one byte each) and the scale of their block
  uint2 kcpre[C::KV_VECS], vcpre[C::KV_VECS];
  unsigned kspre[C::KV_VECS], vspre[C::KV_VECS];
  auto fetch_kv = [&](int kt) {
    const int j0 = kt * N;
    // cache row (of Hkv heads) of key j0's page start, or of the sequence's key 0
    size_t r0 = size_t(b) * seq_rows;
    int jpage0 = 0;  // first key of the tile's page
    if constexpr (EXT) {
      if (p.btab != nullptr) {
        // the table through the constant address space: a scalar load
        typedef const __attribute__((address_space(4))) int* const_int_ptr;
        const const_int_ptr bt = (const_int_ptr)(size_t)(p.btab + size_t(b) * p.max_pages);
        const int pg = min(max(bt[j0 / p.page_size], 0), p.num_pages - 1);
        jpage0 = j0 - j0 % p.page_size;
        r0 = size_t(pg) * p.page_size;
      }
    }
#pragma unroll
    for (int i = 0; i < C::KV_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      const int j = min(j0 + (vid >> 4), T_ - 1);  // rows past T: clamped, masked later
      const size_t row = (r0 + size_t(j - jpage0)) * Hkv + kvh;
      if constexpr (MX) {
        const u8* kc = static_cast<const u8*>(p.k);
        const u8* vc = static_cast<const u8*>(p.v);
        const u8* ksc = static_cast<const u8*>(p.k_scale);
        const u8* vsc = static_cast<const u8*>(p.v_scale);
        kcpre[i] = *reinterpret_cast<const uint2*>(kc + row * D + (vid & 15) * 8);
        vcpre[i] = *reinterpret_cast<const uint2*>(vc + row * D + (vid & 15) * 8);
        kspre[i] = ksc[row * (D / kMxBlock) + (vid & 15) / 4];
        vspre[i] = vsc[row * (D / kMxBlock) + (vid & 15) / 4];
      } else {
        kpre[i] = ld8<T>(kg + row * D + (vid & 15) * 8);
        vpre[i] = ld8<T>(vg + row * D + (vid & 15) * 8);
      }
    }
  };
  u8* Kc = reinterpret_cast<u8*>(Ks);  // MX: K codes [N][kMxKcs], then scales [N][4]
  u8* Ksc = Kc + N * kMxKcs;
  auto store_kv = [&]() {
#pragma unroll
    for (int i = 0; i < C::KV_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      const int row = vid >> 4, c8 = vid & 15;
      if constexpr (MX) {
        *reinterpret_cast<uint2*>(Kc + row * kMxKcs + c8 * 8) = kcpre[i];
        if ((c8 & 3) == 0) Ksc[row * 4 + c8 / 4] = u8(kspre[i]);
        // V codes -> bf16 (exact: a 4-bit significand times a power of two)
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const float sc = e8m0_float(vspre[i]);
        const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vcpre[i].x, sc, false);
        const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vcpre[i].x, sc, true);
        const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vcpre[i].y, sc, false);
        const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vcpre[i].y, sc, true);
        VS::store(Vs, row, c8, v8_t<T>{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]});
      } else {
        st8<T>(Ks + row * C::KS + c8 * 8, kpre[i]);
        VS::store(Vs, row, c8, vpre[i]);
      }
    }
  };
  // MX scores: S^T += K Q^T over d = 64m .. 64m+63 for m = 0, 1 (see the query's layout)
  auto mx_scores = [&](f32x16& acc) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u8* kr = Kc + a * kMxKcs + 64 * m + 16 * h2;
      const uint4 lo = *reinterpret_cast<const uint4*>(kr);
      const uint4 hi = *reinterpret_cast<const uint4*>(kr + 32);
      const i32x8 ka = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      const int ksc = Ksc[a * 4 + 2 * m + h2];
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qx[m], acc, 0, 0, 0, ksc, 0, qsc[m]);
    }
  };

  // P chunk k holds distances [k*N, k*N + N) in ring slot k mod RING.  Vector
  // i of this thread covers chunk row vid/16, columns 8*(vid%16) .. +7.
  // Loads are issued unconditionally from clamped addresses and the zero fill
  // (rows outside [0, E), columns past d_r) is applied when the chunk is
  // stored, so the loads stay in flight until then.  Every column of a slot is
  // written, so the R^T MFMAs always run all kMaxDr/16 k-steps.
  const int vec_per_row = d_r / 8;
  v8_t<T> ppre[C::P_VECS];
  unsigned pok = 0;  // bit i: vector i of the pending chunk holds P values
  auto fetch_p = [&](int k) {
    pok = 0;
#pragma unroll
    for (int i = 0; i < C::P_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      const int d = k * N + (vid >> 4);
      const int c8 = vid & 15;
      pok |= unsigned(d >= 0 && d < E && c8 < vec_per_row) << i;
      ppre[i] = ld8<T>(pcg + size_t(min(max(d, 0), max(E - 1, 0))) * d_r + 8 * min(c8, vec_per_row - 1));
    }
  };
  auto store_p = [&](int k) {
    T* base = Pr + size_t(k & (nqb - 1)) * N * C::PS;
#pragma unroll
    for (int i = 0; i < C::P_VECS; ++i) {
      const int vid = tid + i * C::THREADS;
      st8<T>(base + (vid >> 4) * C::PS + (vid & 15) * 8, ((pok >> i) & 1u) ? ppre[i] : zero8<T>());
    }
  };
  // A chunk is worth staging if some distance in it is below E.
  auto chunk_needed = [&](int k) { return E > 0 && k * N < E && k * N + N > 0; };

  // ---- prologue: first tile and the chunks its waves read
  // Tile kt: the wave's first query is 32c keys after the tile's first key,
  // c = (i0 - 32kt)/32 + qb, so the tile's waves read chunks c0-1 .. c0+nqb-2
  // with c0 = (i0 - 32kt)/32; the ring has nqb slots (chunk k in slot k mod nqb).
  {
    fetch_kv(kt_lo);
    const int c0 = (i0 - kt_lo * N) / N;
    for (int k = c0 - 1; k < c0 - 1 + nqb; ++k) {
      fetch_p(k);
      if (chunk_needed(k)) store_p(k);
    }
    store_kv();
  }

  // Per-wave buffer of relative logits R(a, d) of this wave's queries for the
  // tile's two chunks: chunk c-1 at columns 0..31, chunk c at 32..63, so key
  // b of query a (distance 32c + a - b) is column 32 + a - b.  Chunk c was
  // the new chunk of the previous tile and stays in registers (rprev).
  float* rs = Rs + w * 32 * C::LS;
  f32x16 rprev = zero16();
  int rlast = INT_MIN;  // the chunk rprev holds

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * N;
    const int c0 = (i0 - j0) / N;  // exact: i0 and j0 are multiples of N
    __syncthreads();               // tile kt (K, V and its chunks) is in LDS

    // prefetch tile kt+1 and the one new chunk its waves read (c0 - 2)
    const bool more = kt < kt_hi;
    const int knew = c0 - 2;
    const bool store_new = more && chunk_needed(knew);
    fetch_kv(more ? kt + 1 : kt);
    fetch_p(knew);

    // ---- per-wave work on the (32 queries) x (32 keys) sub-tile
    const bool wdead = qw0 >= T_ || qw0 + 31 < pos0 || j0 > qw0 + 31 || (W > 0 && qw0 - (j0 + N - 1) >= W);
    if (!wdead) {
      const bool wband = E > 0 && max(0, qw0 - (j0 + N - 1)) < E;
      const bool wmask = (j0 + N - 1 > qw0) || (W > 0 && qw0 + 31 - j0 >= W);

      // Scores S^T = K Q^T: lane a's column is query a, accumulator v is key
      // 8*(v/4) + 4*h2 + v%4 of the tile.
      f32x16 s = zero16();
      if (wband) {
        const int c = c0 + qb;
        if (rlast != c) {
          // first tile with bias for this wave: chunk c (its distances may
          // reach below E) straight from P_cols in global memory
          rprev = zero16();
          if (chunk_needed(c)) {
            const int d = c * N + a;
            const bool rok = d >= 0 && d < E;
            const T* prow = pcg + size_t(min(max(d, 0), max(E - 1, 0))) * d_r + 8 * h2;
#pragma unroll
            for (int kk = 0; kk < kMaxDr / 16; ++kk)
              mma32(ld8_or_zero<T>(prow + kk * 16, rok && kk < d_r / 16), rreg[kk], rprev);
          }
        }
        // the new chunk c-1: R^T = P_rows r^T, one MFMA chain beside the QK chain
        f32x16 racc = zero16();
        {
          const T* pr = Pr + ((c - 1) & (nqb - 1)) * (N * C::PS) + a * C::PS + 8 * h2;
          const T* kr = Ks + a * C::KS + 8 * h2;
          if constexpr (MX) mx_scores(s);
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            if constexpr (!MX) mma32(ld8<T>(kr + kk * 16), qreg[kk], s);
            mma32(ld8<T>(pr + kk * 16), rreg[kk], racc);
          }
        }
        // R^T accumulator v is distance 8*(v/4) + 4*h2 + v%4 of its chunk
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float* dst = rs + a * C::LS + 8 * g4 + 4 * h2;
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
        // y = S*(c1/c2) + R(a, 32c + a - b), at column 32 + a - b
        const float* src = rs + a * C::LS + 32 + a - 4 * h2;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = fmaf(s[v], qk_scale, src[-(8 * (v >> 2) + (v & 3))]);
        wave_lds_fence();
      } else if constexpr (MX) {
        mx_scores(s);
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] *= qk_scale;
      } else {
        f32x16 s_odd = zero16();  // two chains keep the matrix cores busy
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const v8_t<T> kf = ld8<T>(Ks + a * C::KS + 8 * h2 + kk * 16);
          if (kk & 1) mma32(kf, qreg[kk], s_odd);
          else mma32(kf, qreg[kk], s);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (s[v] + s_odd[v]) * qk_scale;
      }

      if (wmask) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int dd = qa - (j0 + 8 * (v >> 2) + 4 * h2 + (v & 3));
          if (dd < 0 || (W > 0 && dd >= W)) s[v] = -INFINITY;
        }
      }

      // online softmax (per query = per lane pair l, l^32).  The exponentials
      // are taken against the running maximum first; only when some row
      // maximum grows by more than the lazy margin are O and l rescaled and
      // the exponentials recomputed against the new maximum.
      f32x16 pexp;
      float mx = -INFINITY;
      {
        const float nm = -c2 * m_run;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          mx = fmaxf(mx, s[v]);
          pexp[v] = fast_exp2(fmaf(s[v], c2, nm));
        }
      }
      mx = pair_max32(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_run + lazy) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = fast_exp2(c2 * (m_run - m_new));
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[i][v] *= corr;
        const float nm = -c2 * m_run;
#pragma unroll
        for (int v = 0; v < 16; ++v) pexp[v] = fast_exp2(fmaf(s[v], c2, nm));
      }
      float psum = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) psum += pexp[v];
      l_run += psum;

      // O^T += V^T P^T
#pragma unroll
      for (int c16 = 0; c16 < N / 16; ++c16) {
        v8_t<T> pb;
#pragma unroll
        for (int t = 0; t < 8; ++t) pb[t] = T(pexp[8 * c16 + t]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) mma32(VS::frag(Vs, c16, db, lane), pb, o[db]);
      }
    }

    __syncthreads();  // every wave is done with tile kt's K, V and chunks
    if (more) {
      store_kv();
      if (store_new) store_p(knew);
    }
  }

  // ---- epilogue: normalise, stage the wave's 32 x D output tile in LDS and
  // write it back as whole rows in 16-byte pieces (each lane holds only
  // 4-element fragments of its query's row)
  const float l_tot = pair_sum32(l_run);
  const float inv = 1.0f / l_tot;
  __syncthreads();  // every wave is done with the tile buffers
  constexpr int OS = D + 16 / int(sizeof(T));  // staged row stride (elements)
  static_assert(size_t(WAVES) * 32 * OS * sizeof(T) <= C::LDS_TOTAL, "output staging fits the LDS");
  T* ot = reinterpret_cast<T*>(smem) + size_t(w) * 32 * OS;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      st4_f32<T>(ot + a * OS + db * 32 + g4 * 8 + 4 * h2, o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv,
                 o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
  wave_lds_fence();
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int EPV = 16 / int(sizeof(T));  // elements per 16-byte piece
  constexpr int VPR = D / EPV;              // pieces per row
  static_assert((32 * VPR) % 64 == 0, "whole pieces per lane");
#pragma unroll
  for (int it = 0; it < 32 * VPR / 64; ++it) {
    const int i = lane + 64 * it;
    const int row = i / VPR, cv = i % VPR;
    const int q = qw0 + row;
    if (q >= pos0 && q < T_)
      *reinterpret_cast<u32x4*>(static_cast<T*>(p.out) + (qrow_of(q) * Hq + h) * D + cv * EPV) =
          *reinterpret_cast<const u32x4*>(ot + row * OS + cv * EPV);
  }
  if (p.lse != nullptr && h2 == 0 && qvalid) {
    const size_t li = EXT ? size_t(h) * p.total_q + qrow_of(qa) : (size_t(b) * Hq + h) * T_ + qa;
    p.lse[li] = (c2 * m_run + log2f(l_tot)) * kLn2;
  }
}

template <typename T, int WAVES, bool EXT = false, bool MX = false>
hipError_t launch_prefill_tiles(const PrefillArgs& a, hipStream_t stream) {
  // heads per workgroup: the largest power of two <= WAVES dividing Hq/Hkv
  const int G = a.Hq / a.Hkv;
  int hpw = 1;
  while (hpw * 2 <= WAVES && G % (hpw * 2) == 0) hpw *= 2;
  const int M = 32 * (WAVES / hpw);
  // extend: the tiles of a sequence cover max_q rows at any alignment
  const int n_qt = EXT ? (a.max_q + M - 1) / M + 1 : (a.T + M - 1) / M;
  const long long n_items = (long long)n_qt * a.B * a.Hkv * (G / hpw);
  if (n_items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (n_items == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_kernel<T, WAVES, EXT, MX>), dim3((unsigned)n_items),
                     dim3(PrefillCfg<T, WAVES>::THREADS), 0, stream, a, n_qt, (int)n_items, hpw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16, Hq/Hkv a multiple of 8: the eight waves of a workgroup are eight query
// heads of one kv head on the same 32 queries (one K, V and P tile serves all
// of them), and the next tile streams into LDS by DMA while this one computes.
//
// global_load_lds_dwordx4 writes each lane's 16 bytes at M0 + 16*lane, so a
// wave instruction fills 1 KB = four 256-byte tile rows.  Lanes choose their
// source chunk so that a row's 16-byte chunks land XOR-swizzled: chunk q of
// row r sits at slot q ^ sw(r), with sw(r) = r & 7 for K and P (the 8 lanes of
// a 16-byte fragment read hit 8 distinct bank groups) and sw(r) = 2*(r & 3)
// for V (the 16 lanes of a transpose read cover the 32 banks once).
//
// The tile loop is software-pipelined inside each wave: one iteration runs
// the scores and relative logits of tile t+1, the softmax of tile t and the
// PV product of tile t-1 in one straight-line block, so the matrix cores
// work while the VALU runs tile t's exponentials.  LDS holds K and P of tile
// t+1 and V of tile t-1; the DMA fills K and P of tile t+2 and V of tile t
// (all double-buffered by tile parity, one barrier per tile).  The loop is
// unrolled by two so every LDS address is a per-lane offset plus a constant.
// P rows for distances outside [0, E) are DMA'd from a zero row.
// ---------------------------------------------------------------------------
struct DmaCfg {
  static constexpr int N = 32;
  static constexpr int ROWB = kHeadDim * 2;  // bytes per K / V / P tile row (d_r padded to 128)
  static constexpr int TILEB = N * ROWB;     // 8 KB
  static constexpr int LS = 3 * N + 4;       // R buffer row stride (floats): three chunk slots + 4
  static constexpr int THREADS = 512;
  static constexpr size_t OFF_K = 0, OFF_V = 2 * TILEB, OFF_P = 4 * TILEB, OFF_R = 6 * TILEB;
  static constexpr size_t LDS_TOTAL = OFF_R + size_t(8) * 32 * LS * sizeof(float);
  static_assert(kMaxDr == kHeadDim, "P rows share the K tile geometry");
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// M0 (the DMA's LDS base) is saved and restored around the load, so the
// compiler's own use of M0 is untouched.
__device__ __forceinline__ void dma16(const void* src, unsigned lds_base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}
// The same with a uniform 64-bit base and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(const void* base, unsigned off, unsigned lds_base) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A zero P row: DMA source for distances outside [0, E), so their relative
// logits come out zero without a test.
__device__ __attribute__((aligned(16))) const __bf16 kZeroPRow[kMaxDr] = {};

template <int V> struct IntC { static constexpr int value = V; };

// A use of x at this point: the code that makes x stays ahead of a following
// branch instead of being moved past it (the work then overlaps the matrix
// instructions before the branch).
template <typename X>
__device__ __forceinline__ void materialize(const X& x) {
  asm volatile("" ::"v"(x));
}

// v_max3_f32 without the quieting of NaN inputs that fmaxf implies (callers
// pass no NaN)
__device__ __forceinline__ float max3_f32(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

// RAWQK (alpha > 0): tiles without bias keep the raw scores q.k; the row
// maximum is scaled once and the exponent takes c1 = s*alpha*log2(e) in
// place of c2, which saves a multiply per score (and one of two score
// accumulation chains).
// EXT: 0 prefill; 1 and 2 the extend form (rel_attn_extend) over a
// contiguous (1) or paged (2, power-of-two page size) cache.
template <bool RAWQK, int EXT = 0>
__global__ __launch_bounds__(512, 1) void prefill_dma_kernel(PrefillArgs p, int n_qt, int n_items) {
  using C = DmaCfg;
  using T = __bf16;
  constexpr int N = C::N;
  constexpr int D = kHeadDim;

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_TOTAL];
  float* const Rs = reinterpret_cast<float*>(smem + C::OFF_R);

  const int Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;
  const int d_r = p.d_r, E = p.E, W = p.W;

  // ---- workgroup -> (32-query tile, batch, kv head, group of 8 heads),
  // longest query tiles first
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int n_hs = G / 8;
  const int per_qt = p.B * Hkv * n_hs;
  const int qt = n_qt - 1 - item / per_qt;
  int rest = item % per_qt;
  const int hs = rest % n_hs;
  rest /= n_hs;
  const int kvh = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int a = lane & 31;
  const int h = kvh * G + hs * 8 + w;

  // T_: keys (and positions) of this sequence.  Extend: its new rows are
  // positions [pos0, T_), packed from row row0 of q, r and out; query tiles
  // are aligned to 32 in positions, so the distance chunks are those of a
  // prefill, and rows before pos0 are neither loaded nor stored.
  int T_ = p.T, pos0 = 0, row0 = 0, qt_abs = qt;
  float c1 = p.c1, c2 = p.c2;
  if constexpr (EXT != 0) {
    const int cap = EXT == 2 ? p.max_pages * p.page_size : p.cap;
    T_ = max(0, min(p.kv_len[b], cap));
    row0 = min(max(p.q_start[b], 0), p.total_q);
    const int n = max(0, min(min(p.q_start[b + 1] - p.q_start[b], min(T_, p.max_q)), p.total_q - row0));
    pos0 = T_ - n;
    qt_abs = pos0 / N + qt;
    if (n == 0 || qt_abs * N >= T_) return;
    if (p.log_scale) {  // s = max(1, ln(kv_len) / ln(4096)), one per sequence
      const float sc = fmaxf(1.0f, logf(float(T_)) * (1.0f / 8.317766166719343f));
      c2 = sc * 1.4426950408889634f;
      c1 = c2 * p.alpha;
    }
  }
  const int q0 = qt_abs * N;
  const int qa = q0 + a;
  const bool qvalid = qa >= pos0 && qa < T_;
  // packed row of query position x (prefill: b*T + x)
  auto qrow_of = [&](int x) -> size_t {
    if constexpr (EXT != 0) return size_t(row0 + x - pos0);
    else return size_t(b) * T_ + x;
  };

  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  const T* rg = static_cast<const T*>(p.r);
  const T* pcg = E > 0 ? static_cast<const T*>(p.pc) : kg;

  const float qk_scale = c1 / c2;

  bf16x8 qreg[D / 16];
  {
    const T* qrow = qg + (qrow_of(qvalid ? qa : pos0) * Hq + h) * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = ld8_or_zero<T>(qrow + kk * 16, qvalid);
  }
  bf16x8 rreg[kMaxDr / 16];  // zero past d_r
  {
    const int nkr = d_r / 16;
    const T* rrow = rg + (qrow_of(qvalid ? qa : pos0) * Hq + h) * d_r + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) rreg[kk] = ld8_or_zero<T>(rrow + kk * 16, E > 0 && qvalid && kk < nkr);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();

  const int i_last = min(q0 + N - 1, T_ - 1);
  const int kt_lo = W > 0 ? max(0, q0 - W + 1) / N : 0;
  const int kt_hi = i_last / N;

  // ---- DMA: this wave fills rows 4w .. 4w+3 of a K, V or P tile; lane l
  // writes slot l%16 of row 4w + l/16
  const int drow = 4 * w + (lane >> 4);
  const int dslot = lane & 15;
  const int qk_src = dslot ^ (drow & 7);        // K / P chunk landing in this slot
  const int qv_src = dslot ^ (2 * (drow & 3));  // V chunk landing in this slot
  // K and V rows of this sequence and kv head: a uniform base advanced to the
  // tile's first row plus a 32-bit byte offset per lane, clamped to the
  // sequence's last row (prefill: the host keeps T*Hkv*D*2 below 2^31).
  // Extend: row b*cap + j of a contiguous cache, or slot j % page_size of
  // page btab[b][j / page_size] (a tile lies in one page; page ids clamped
  // to the pool).
  const T* kseq = kg + (EXT != 0 ? size_t(kvh) : (size_t(b) * T_ * Hkv + kvh)) * D;
  const T* vseq = vg + (EXT != 0 ? size_t(kvh) : (size_t(b) * T_ * Hkv + kvh)) * D;
  const unsigned rowb = unsigned(Hkv) * D * 2;
  const int page_shift = EXT == 2 ? __builtin_ctz(unsigned(p.page_size)) : 0;
  const unsigned drow_b = unsigned(drow) * rowb;
  const unsigned kcol = 16u * unsigned(qk_src), vcol = 16u * unsigned(qv_src);
  const unsigned pcol = 16u * unsigned(min(qk_src, d_r / 8 - 1));
  const T* const zrow = kZeroPRow + 8 * qk_src;
  const unsigned lds0 = unsigned(reinterpret_cast<size_t>(smem)) + 1024u * unsigned(w);
  auto chunk0 = [&](int kt) { return (q0 - kt * N) / N; };
  // page of tile kt (paged extend; 0 otherwise)
  // (the table is read through the constant address space: scalar loads,
  // which the vector-memory wait closing each iteration does not count)
  typedef const __attribute__((address_space(4))) int* const_int_ptr;
  const_int_ptr btab_row = EXT == 2 ? (const_int_ptr)(size_t)(p.btab + size_t(b) * p.max_pages) : nullptr;
  auto page_of = [&](int kt) {
    if constexpr (EXT == 2) return min(max(btab_row[(kt * N) >> page_shift], 0), p.num_pages - 1);
    else return 0;
  };
  // address of tile kt's first row; pg = page_of(kt), looked up ahead of
  // time by the loop (a scalar load waited for at the DMA issue would stall
  // the issuing waves every tile)
  auto tile_base = [&](const T* seq, int kt, int pg) {
    const int j0 = kt * N;
    if constexpr (EXT == 0) {
      return reinterpret_cast<const T*>(reinterpret_cast<const char*>(seq) + size_t(unsigned(j0) * rowb));
    } else {
      size_t row = size_t(b) * p.cap + j0;  // cache row of the tile's first key
      if constexpr (EXT == 2) row = (size_t(pg) << page_shift) + (j0 & (p.page_size - 1));
      return reinterpret_cast<const T*>(reinterpret_cast<const char*>(seq) + row * rowb);
    }
  };
  auto lane_off = [&](int kt, unsigned col) { return min(drow_b, unsigned(T_ - 1 - kt * N) * rowb) + col; };
  // K of tile kt (kt <= kt_hi) into K buffer buf
  auto issue_k = [&](int kt, int buf, int pg) {
    dma16s(tile_base(kseq, kt, pg), lane_off(kt, kcol), __builtin_amdgcn_readfirstlane(lds0 + C::OFF_K + buf * C::TILEB));
  };
  // tile kt's new distance chunk of P rows into P buffer buf
  auto issue_p = [&](int kt, int buf) {
    const int d = (chunk0(kt) - 1) * N + drow;
    const T* src = unsigned(d) < unsigned(E)
                       ? reinterpret_cast<const T*>(reinterpret_cast<const char*>(pcg) + unsigned(d) * unsigned(2 * d_r) + pcol)
                       : zrow;
    dma16(src, __builtin_amdgcn_readfirstlane(lds0 + C::OFF_P + buf * C::TILEB));
  };
  // V of tile kt into V buffer kt & 1
  auto issue_v = [&](int kt, int pg) {
    dma16s(tile_base(vseq, kt, pg), lane_off(kt, vcol), __builtin_amdgcn_readfirstlane(lds0 + C::OFF_V + (kt & 1) * C::TILEB));
  };
  // K and V of a plain iteration, issued by waves 0-3 alone (eight rows each).
  // Measured with per-wave cycle counters on the 32K shape: waves 0-3 reach
  // the next barrier about 300 cycles per tile before waves 4-7 (their SIMD
  // partners) and wait there, so they take over the partners' DMA work.
  const int erow = 8 * (w & 3) + (lane >> 4);
  const unsigned erow_b0 = unsigned(erow) * rowb, erow_b1 = unsigned(erow + 4) * rowb;
  const unsigned ekcol0 = 16u * unsigned(dslot ^ (erow & 7)), ekcol1 = 16u * unsigned(dslot ^ ((erow + 4) & 7));
  const unsigned evcol = 16u * unsigned(dslot ^ (2 * (erow & 3)));
  const unsigned elds = unsigned(reinterpret_cast<size_t>(smem)) + 2048u * unsigned(w & 3);
  auto issue_kv4 = [&](int ktk, int buf, int ktv, int pgk, int pgv) {
    if (w < 4) {
      const unsigned limk = unsigned(T_ - 1 - ktk * N) * rowb, limv = unsigned(T_ - 1 - ktv * N) * rowb;
      const unsigned lk = __builtin_amdgcn_readfirstlane(elds + C::OFF_K + buf * C::TILEB);
      const unsigned lv = __builtin_amdgcn_readfirstlane(elds + C::OFF_V + (ktv & 1) * C::TILEB);
      dma16s(tile_base(kseq, ktk, pgk), min(erow_b0, limk) + ekcol0, lk);
      dma16s(tile_base(kseq, ktk, pgk), min(erow_b1, limk) + ekcol1, lk + 1024);
      dma16s(tile_base(vseq, ktv, pgv), min(erow_b0, limv) + evcol, lv);
      dma16s(tile_base(vseq, ktv, pgv), min(erow_b1, limv) + evcol, lv + 1024);
    }
  };
  auto band_of = [&](int kt) { return E > 0 && max(0, q0 - (kt * N + N - 1)) < E; };
  // K and, for a tile with bias, its P chunk (buffer kt & 1)
  auto issue_kp = [&](int kt) {
    issue_k(kt, kt & 1, page_of(kt));
    if (band_of(kt)) issue_p(kt, kt & 1);
  };
  // A tile needs the mask when it holds a key past one of its queries (tile
  // qt, the diagonal, and beyond) or one at least W before a query (tiles up
  // to m_lo): one unsigned comparison.
  const int m_lo = (W > 0 && q0 + 31 - W >= 0) ? (q0 + 31 - W) / N : -1;
  auto mask_of = [&](int kt) { return unsigned(kt - m_lo - 1) >= unsigned(qt_abs - m_lo - 1); };
  // Lane byte offsets of the MFMA fragments.  K / P A-operand of k-step kk:
  // row a, chunk (h2 + 2kk) ^ (a & 7); k-steps kk and kk+4 are 128 bytes
  // apart (chunk bit 3 lies outside the swizzle).
  int offkp[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offkp[kk] = a * C::ROWB + (((h2 + 2 * kk) ^ (a & 7)) << 4);
  auto frag_kp = [&](const unsigned char* t, int kk) {
    return ld8<T>(reinterpret_cast<const T*>(t + offkp[kk & 3] + 128 * (kk >> 2)));
  };
  // V transpose reads (PreV<__bf16> layout with V's swizzle): lane (G, s)
  // reads rows 16*c16 + 4*(G/2) + s/4 (+8), columns 32*db + 16*(G%2) +
  // 4*(s%4): chunk 4*db + 2*(G%2) + (s%4)/2, half s%2.  Column blocks db and
  // db+2 are 128 bytes apart.
  int offv[2];
  {
    const int Gq = lane >> 4, sq = lane & 15;
    const int vsw = 2 * ((sq >> 2) & 3);  // rows r and r+8 share r & 3 = s/4
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int q = 4 * db + 2 * (Gq & 1) + ((sq & 3) >> 1);
      offv[db] = (4 * (Gq >> 1) + (sq >> 2)) * C::ROWB + ((sq & 1) << 3) + ((q ^ vsw) << 4);
    }
  }

  // Per-wave relative-logit buffer [query][distance].  The chunk made on
  // tile t (its new chunk, distances 32(c-1) .. 32c-1 with c = qt - t) sits
  // at columns 32*(t&1), and chunks of even t also at 64..95, so tile t's
  // chunks c-1 and c are 64 contiguous columns from 32*(t&1) and each tile
  // writes only its new chunk; key b of query a (distance 32c + a - b) is
  // column 32*(t&1) + 32 + a - b.  R^T accumulator v is distance
  // 8*(v/4) + 4*h2 + v%4 of its chunk.
  float* const rs = Rs + w * 32 * C::LS;
  float* const rput = rs + a * C::LS + 4 * h2;
  const float* const rsh = rs + a * (C::LS + 1) + 32 - 4 * h2;
  auto put_chunk = [&](int t, const f32x16& acc) {
    float* const dst = rput + 32 * (t & 1);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[4 * g4 + e];
      *reinterpret_cast<f32x4*>(dst + 8 * g4) = x;
      if ((t & 1) == 0) *reinterpret_cast<f32x4*>(dst + 64 + 8 * g4) = x;
    }
  };
  // First tile t with bias: chunk c0 (made, by the rule above, on tile t-1)
  // straight from P_cols in global memory.
  auto first_chunk = [&](int t) {
    const int c0 = chunk0(t);
    const int d = c0 * N + a;
    const bool rok = d >= 0 && d < E;
    const int nk = d_r / 16;
    const T* prow = pcg + size_t(min(max(d, 0), E - 1)) * d_r + 8 * h2;
    bf16x8 pf[kMaxDr / 16];
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) pf[kk] = ld8<T>(prow + min(kk, nk - 1) * 16);
    f32x16 rc = zero16();
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) mma32((rok && kk < nk) ? pf[kk] : zero8<T>(), rreg[kk], rc);
    put_chunk(t - 1, rc);
  };
  // s <- s*(c1/c2) + bias along the shear, once tile t's new chunk is stored
  auto shear_add = [&](int t, f32x16& s) {
    wave_lds_fence();
    const float* src = rsh + 32 * (t & 1);
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = fmaf(s[v], qk_scale, src[-(8 * (v >> 2) + (v & 3))]);
  };
  auto apply_mask = [&](int kt, f32x16& s) {
    const int j0 = kt * N;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int dd = qa - (j0 + 8 * (v >> 2) + 4 * h2 + (v & 3));
      if (dd < 0 || (W > 0 && dd >= W)) s[v] = -INFINITY;
    }
  };
  // p = exp2(c2*y - c2*m), its row sum, and the bf16 PV operand
  auto exps = [&](const f32x16& s, float cs, float nm, bf16x8 (&pb)[2], float& psum) {
    f32x16 pe;
#pragma unroll
    for (int v = 0; v < 16; ++v) pe[v] = fast_exp2(fmaf(s[v], cs, nm));
    float s8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) s8[v] = pe[2 * v] + pe[2 * v + 1];
    psum = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
#pragma unroll
    for (int c16 = 0; c16 < 2; ++c16)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[c16][t] = T(pe[8 * c16 + t]);
  };
  // O^T += V^T P^T
  auto pv = [&](const unsigned char* vt_b, const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int c16 = 0; c16 < N / 16; ++c16) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const T* p0 = reinterpret_cast<const T*>(vt_b + 16 * c16 * C::ROWB + offv[db & 1] + 128 * (db >> 1));
        const s16x4 x = lds_read_tr(p0);
        const s16x4 y = lds_read_tr(p0 + 8 * (C::ROWB / 2));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
        mma32(vf, pb[c16], o[db]);
      }
    }
  };

  // ---- prologue: tile kt_lo's K (and P) in LDS, its scores, K and P of tile
  // kt_lo+1 in flight.  The compiler-visible wait also retires the q and r
  // loads, so no wait for them lands inside the tile loop.  The V buffer that
  // the first iteration's PV reads (the tile before kt_lo) is zeroed, so that
  // product adds nothing.
  issue_kp(kt_lo);
  {
    typedef unsigned u32x4z __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4z*>(smem + C::OFF_V + ((kt_lo + 1) & 1) * C::TILEB + 16 * tid) = u32x4z{0, 0, 0, 0};
  }
  dma_wait();
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  if (kt_lo < kt_hi) issue_kp(kt_lo + 1);
  f32x16 s_cur = zero16();
  {
    const unsigned char* kt_b = smem + C::OFF_K + (kt_lo & 1) * C::TILEB;
    const unsigned char* pt_b = smem + C::OFF_P + (kt_lo & 1) * C::TILEB;
    if (band_of(kt_lo)) {
      first_chunk(kt_lo);
      f32x16 racc = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        mma32(frag_kp(kt_b, kk), qreg[kk], s_cur);
        mma32(frag_kp(pt_b, kk), rreg[kk], racc);
      }
      put_chunk(kt_lo, racc);
      shear_add(kt_lo, s_cur);
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) mma32(frag_kp(kt_b, kk), qreg[kk], s_cur);
      if constexpr (!RAWQK) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s_cur[v] *= qk_scale;
      }
    }
    if (mask_of(kt_lo)) apply_mask(kt_lo, s_cur);
  }
  // scores of tile kt are raw (units of q.k) when it has no bias
  auto raw_of = [&](int kt) { return RAWQK && !band_of(kt); };
  // row maximum of a score tile in units of c2 (scores are never NaN:
  // v_max3 without the quieting of fmaxf)
  auto row_max = [&](const f32x16& s, bool raw) {
    const float m0 = max3_f32(s[0], s[1], s[2]), m1 = max3_f32(s[3], s[4], s[5]);
    const float m2 = max3_f32(s[6], s[7], s[8]), m3 = max3_f32(s[9], s[10], s[11]);
    const float m5 = max3_f32(s[12], s[13], s[14]);
    float mx = max3_f32(max3_f32(m0, m1, m2), max3_f32(m3, m5, s[15]), -INFINITY);
    const unsigned u = __float_as_uint(mx);
    const auto r2 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    mx = max3_f32(__uint_as_float(r2[0]), __uint_as_float(r2[1]), -INFINITY);
    return raw ? mx * qk_scale : mx;
  };
  // The running maximum starts at tile kt_lo's and is raised only when a
  // tile's exponentials (taken against it) sum past kPsumLimit on some lane:
  // then the tile's true maximum is taken, O and l are rescaled and the
  // exponentials redone.  Below the limit every p is at most kPsumLimit, so
  // nothing overflows; the result is exact either way.
  float m_run = fmaxf(row_max(s_cur, raw_of(kt_lo)), -1e30f);
  float l_run = 0.0f;
  dma_wait();

  // ---- tile loop.  Iteration kt runs, in one straight-line block, the
  // scores of tile kt+1, the softmax of tile kt and the PV product of tile
  // kt-1 (whose p it kept), so the matrix cores have independent work while
  // the VALU runs the exponentials.  LDS holds K and P of tile kt+1 and V of
  // tile kt-1; the DMA fills K and P of tile kt+2 and V of tile kt.  Tiles
  // with bias are a suffix of the range (the keys nearest the queries), so
  // the loop runs in two parts; the last tile is peeled, and each part is
  // unrolled by two so every LDS address is a lane offset plus a constant
  // and the p of consecutive tiles alternate between two register sets.
  bf16x8 pbt[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) pbt[i][0] = pbt[i][1] = zero8<T>();
  // pages of the K tile and the V tile the next iteration loads
  int pg_k = page_of(min(kt_lo + 2, kt_hi)), pg_v = page_of(kt_lo);
  // Each iteration starts with a barrier (K/P of tile kt+1 and V of tile
  // kt-1 are in LDS; all waves are past iteration kt-1) and issues its DMA
  // without a branch: past the last tile, tile kt_hi is loaded again into the
  // free buffer.  P chunks are loaded only by iterations whose next tile has
  // bias; the first tile with bias that a plain iteration would have loaded
  // gets its chunk between the two parts of the loop.
  // the (rare) raise of the running maximum; pb and psum are redone
  auto settle = [&](const f32x16& s, bool raw, float cs, bf16x8 (&pb)[2], float& psum) {
    if (__builtin_amdgcn_ballot_w64(psum > kPsumLimit) != 0) {
      const float m_new = fmaxf(m_run, row_max(s, raw));
      const float corr = fast_exp2(c2 * (m_run - m_new));
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= corr;
      exps(s, cs, -c2 * m_run, pb, psum);
    }
    l_run += psum;
  };
  // one iteration whose next tile has no bias; PAR = kt & 1
  auto plain_step = [&](auto par, f32x16& s, f32x16& s_nx, int kt) {
    constexpr int PAR = decltype(par)::value, NP = PAR ^ 1;
    __syncthreads();
    // pages for the next iteration, loaded ahead of this iteration's DMA
    // (both end at its closing wait)
    const int pgk_n = page_of(min(kt + 3, kt_hi)), pgv_n = page_of(kt + 1);
    issue_kv4(min(kt + 2, kt_hi), PAR, kt, pg_k, pg_v);
    pg_k = pgk_n;
    pg_v = pgv_n;
    constexpr bool raw = RAWQK;  // tiles before the band have no bias
    const float cs = raw ? c1 : c2;
    const float nm = -c2 * m_run;
    const unsigned char* kt_b = smem + C::OFF_K + NP * C::TILEB;
    const unsigned char* vt_b = smem + C::OFF_V + NP * C::TILEB;
    float psum;
    if constexpr (RAWQK) {  // raw scores of tile kt+1: one chain, no scaling
      s_nx = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) mma32(frag_kp(kt_b, kk), qreg[kk], s_nx);
      exps(s, cs, nm, pbt[PAR], psum);
      pv(vt_b, pbt[NP]);
    } else {
      f32x16 s_odd = zero16();
      s_nx = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 kf = frag_kp(kt_b, kk);
        if (kk & 1) mma32(kf, qreg[kk], s_odd);
        else mma32(kf, qreg[kk], s_nx);
      }
      exps(s, cs, nm, pbt[PAR], psum);
      pv(vt_b, pbt[NP]);
#pragma unroll
      for (int v = 0; v < 16; ++v) s_nx[v] = (s_nx[v] + s_odd[v]) * qk_scale;
    }
    materialize(pbt[PAR][0]);
    materialize(pbt[PAR][1]);
    settle(s, raw, cs, pbt[PAR], psum);
    if (mask_of(kt + 1)) apply_mask(kt + 1, s_nx);
    dma_wait();  // this wave's parts of the next tiles have landed
  };
  // one iteration whose next tile has bias
  auto band_step = [&](auto par, f32x16& s, f32x16& s_nx, int kt) {
    constexpr int PAR = decltype(par)::value, NP = PAR ^ 1;
    __syncthreads();
    const int kn = min(kt + 2, kt_hi);
    const int pgk_n = page_of(min(kt + 3, kt_hi)), pgv_n = page_of(kt + 1);  // next iteration's pages
    issue_k(kn, PAR, pg_k);
    issue_p(kn, PAR);
    issue_v(kt, pg_v);
    pg_k = pgk_n;
    pg_v = pgv_n;
    const bool raw = raw_of(kt);
    const float cs = raw ? c1 : c2;
    const float nm = -c2 * m_run;
    const unsigned char* kt_b = smem + C::OFF_K + NP * C::TILEB;
    const unsigned char* pt_b = smem + C::OFF_P + NP * C::TILEB;
    const unsigned char* vt_b = smem + C::OFF_V + NP * C::TILEB;
    f32x16 racc = zero16();
    s_nx = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) mma32(frag_kp(pt_b, kk), rreg[kk], racc);
    put_chunk(NP, racc);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) mma32(frag_kp(kt_b, kk), qreg[kk], s_nx);
    float psum;
    exps(s, cs, nm, pbt[PAR], psum);
    pv(vt_b, pbt[NP]);
    shear_add(NP, s_nx);
    materialize(pbt[PAR][0]);
    materialize(pbt[PAR][1]);
#pragma unroll
    for (int v = 0; v < 16; ++v) materialize(s_nx[v]);
    settle(s, raw, cs, pbt[PAR], psum);
    if (mask_of(kt + 1)) apply_mask(kt + 1, s_nx);
    dma_wait();  // this wave's parts of the next tiles have landed
  };
  f32x16 s_b;
  int kt = kt_lo;
  // iterations kt .. kt_end-1, scores in s_cur at entry and exit
  auto run = [&](auto step, int kt_end) {
    if ((kt & 1) && kt < kt_end) {
      step(IntC<1>{}, s_cur, s_b, kt);
      s_cur = s_b;
      ++kt;
    }
    for (; kt + 1 < kt_end; kt += 2) {
      step(IntC<0>{}, s_cur, s_b, kt);
      step(IntC<1>{}, s_b, s_cur, kt + 1);
    }
    if (kt < kt_end) {
      step(IntC<0>{}, s_cur, s_b, kt);
      s_cur = s_b;
      ++kt;
    }
  };
  const int kt_band = E > 0 ? max(kt_lo, (q0 - E + 1) / N) : kt_hi + 1;  // first tile with bias
  run(plain_step, min(kt_hi, kt_band - 1));
  if (kt_band >= kt_lo + 2 && kt_band <= kt_hi) {
    issue_p(kt_band, kt_band & 1);
    dma_wait();
  }
  if (kt < kt_hi && !band_of(kt_lo)) first_chunk(kt + 1);
  run(band_step, kt_hi);
  // the last tile: its softmax with the PV of the one before, then its own PV
  auto last_tile = [&](auto par) {
    constexpr int PAR = decltype(par)::value, NP = PAR ^ 1;
    __syncthreads();
    issue_v(kt, pg_v);
    const bool raw = raw_of(kt);
    const float cs = raw ? c1 : c2;
    float psum;
    exps(s_cur, cs, -c2 * m_run, pbt[PAR], psum);
    pv(smem + C::OFF_V + NP * C::TILEB, pbt[NP]);
    settle(s_cur, raw, cs, pbt[PAR], psum);
    dma_wait();
    __syncthreads();
    pv(smem + C::OFF_V + PAR * C::TILEB, pbt[PAR]);
  };
  if (kt & 1) last_tile(IntC<1>{});
  else last_tile(IntC<0>{});

  // ---- epilogue: normalise, stage the wave's 32 x D tile in LDS, write whole
  // rows in 16-byte pieces
  const float l_tot = pair_sum32(l_run);
  const float inv = 1.0f / l_tot;
  __syncthreads();
  constexpr int OS = D + 8;
  static_assert(size_t(8) * 32 * OS * sizeof(T) <= C::LDS_TOTAL, "output staging fits the LDS");
  T* ot = reinterpret_cast<T*>(smem) + size_t(w) * 32 * OS;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      st4_f32<T>(ot + a * OS + db * 32 + g4 * 8 + 4 * h2, o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv,
                 o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
  wave_lds_fence();
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int i = lane + 64 * it;
    const int row = i >> 4, cv = i & 15;
    const int q = q0 + row;
    if (q >= pos0 && q < T_)
      *reinterpret_cast<u32x4*>(static_cast<T*>(p.out) + (qrow_of(q) * Hq + h) * D + cv * 8) =
          *reinterpret_cast<const u32x4*>(ot + row * OS + cv * 8);
  }
  if (p.lse != nullptr && h2 == 0 && qvalid) {
    const size_t li = EXT != 0 ? size_t(h) * p.total_q + qrow_of(qa) : (size_t(b) * Hq + h) * T_ + qa;
    p.lse[li] = (c2 * m_run + log2f(l_tot)) * kLn2;
  }
}

template <int EXT>
hipError_t launch_prefill_dma(const PrefillArgs& a, hipStream_t stream) {
  // extend: the tiles of a sequence cover max_q rows at any alignment
  const int n_qt = EXT != 0 ? (a.max_q + 31) / 32 + 1 : (a.T + 31) / 32;
  const long long n_items = (long long)n_qt * a.B * a.Hkv * (a.Hq / a.Hkv / 8);
  if (n_items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (n_items == 0) return hipSuccess;
  if (a.c1 > 0.0f)
    hipLaunchKernelGGL((prefill_dma_kernel<true, EXT>), dim3((unsigned)n_items), dim3(DmaCfg::THREADS), 0, stream, a,
                       n_qt, (int)n_items);
  else
    hipLaunchKernelGGL((prefill_dma_kernel<false, EXT>), dim3((unsigned)n_items), dim3(DmaCfg::THREADS), 0, stream,
                       a, n_qt, (int)n_items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_extend(int dtype, const PrefillArgs& a, hipStream_t stream) {
  if (dtype == 1) {
    // the DMA kernel for eight or more query heads per kv head (P addressed
    // with 32-bit offsets; a paged cache with a power-of-two page size)
    const bool dma = (a.Hq / a.Hkv) % 8 == 0 && (long long)a.E * a.d_r * 2 < (1LL << 31);
    if (dma && a.btab == nullptr) return launch_prefill_dma<1>(a, stream);
    if (dma && (a.page_size & (a.page_size - 1)) == 0) return launch_prefill_dma<2>(a, stream);
    return launch_prefill_tiles<__bf16, 8, true>(a, stream);
  }
  return launch_prefill_tiles<float, 2, true>(a, stream);
}

hipError_t launch_extend_mx(const PrefillArgs& a, hipStream_t stream) {
  static_assert(kMxKcs * 32 + 32 * 4 <= PrefillCfg<__bf16, 8>::LDS_K, "MXFP8 K tile fits the K tile's LDS");
  return launch_prefill_tiles<__bf16, 8, true, true>(a, stream);
}

hipError_t launch_prefill(int dtype, const PrefillArgs& a, hipStream_t stream) {
  if (dtype == 1) {
    // The DMA kernel addresses one sequence's K / V rows and P with 32-bit
    // byte offsets.
    const bool offsets32 = (long long)a.T * a.Hkv * kHeadDim * 2 < (1LL << 31) &&
                           (long long)a.E * a.d_r * 2 < (1LL << 31);
    if ((a.Hq / a.Hkv) % 8 == 0 && offsets32) return launch_prefill_dma<0>(a, stream);
    return launch_prefill_tiles<__bf16, 8>(a, stream);
  }
  return launch_prefill_tiles<float, 2>(a, stream);
}

}  // namespace relattn
