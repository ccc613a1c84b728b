// Relative-attention decode for gfx950: one query token per sequence at
// position L-1 against a KV cache [B, L, Hkv, D].
//
// The logit is the one of page "SGLang and Miles Add Day-0 Support for
// Inkling", section "Attention with Relative Positional Embedding"; for the
// single query i = L-1 the bias of key j is s * r.P[:, L-1-j] when
// L-1-j < E.  The visible keys (all of them, or the last `window`) are cut
// into num_splits contiguous chunks (the split-KV "num_splits" of the vLLM
// page, section on the sheared-bias FA4 kernel; the first chunks a few
// quanta longer than the last, which also makes the bias); each workgroup owns one
// (sequence, split, kv head, group of up to 16 query heads), its waves take
// interleaved 32-key steps, and it streams its chunk of K and V exactly once
// for every query head of the group.  The
// partial softmax states (unnormalised o, running max m, sum l) go to the
// caller's workspace and a second kernel merges them by log-sum-exp (with
// a single split the workgroup normalises and writes the output itself).
//
// Two launches on the caller's stream (three when the bias takes the
// pre-pass):
//   1. decode_split_kernel: the workgroups whose split holds keys within E
//      of the query first make the bias s * log2(e) * r.P[:, L-1-j] of those
//      keys and their query heads with MFMAs into LDS (a single query needs
//      no shear).  Per 32-key step a wave computes S^T = K Q^T with
//      16x16x32 MFMAs (rows = keys, columns = query heads, padded to 16),
//      adds the bias of its keys from LDS, applies the online softmax and
//      accumulates O^T = V^T P^T.  The
//      wave keeps two 32-key steps of K and V in flight in registers
//      (ping-pong, no copies), so HBM latency overlaps the previous step's
//      work.  V goes through a wave-private LDS tile: bf16 tiles are stored
//      row-major and read as MFMA fragments with the gfx950 transpose read
//      (ds_read_b64_tr_b16); fp32 tiles are stored transposed.
//      Pre-pass form, when the bias region would not fit the LDS budget:
//      rel_logits_kernel first writes, per (sequence, query head), the bias
//      row for the last E distances into the workspace, stored reversed so
//      that key j reads entry j - L + rl_base and entries beyond E are zero,
//      and the split kernel loads its keys' entries with each step.
//   2. decode_merge_kernel: log-sum-exp merge of the split partials.
#include "device_common.hpp"
#include "mx_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecKeys = 32;  // keys per step
constexpr int kDecDepth = 2;  // steps in flight per wave (a ring of register buffers)
// Keys per split are a multiple of this: every wave of the workgroup runs the
// same whole number of ring turns.
constexpr int kDecSplitQuantum = kDecWaves * kDecKeys * kDecDepth;
constexpr float kLazyRescale = 8.0f;  // log2 units: p may reach 2^8 before O is rescaled

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)((__attribute__((address_space(3))) void*)p)));
}

// V staging.  k-slot 8*g + t of the PV MFMA (lane group g = lane/16) holds
// key 4*g + t (t < 4) or 16 + 4*g + (t-4) (t >= 4): the keys lane (g, c)
// holds in its two S^T accumulators.  Lane (g, c) loaded keys 8g..8g+7, d-chunk c.
template <typename T> struct DecV;

template <> struct DecV<__bf16> {
  // Row-major [32 keys][144]: 288-byte rows put the 8 rows a half-wave
  // transpose read touches in 8 distinct 32-byte bank groups.
  static constexpr int ROW = 144;
  static constexpr size_t BYTES = size_t(kDecKeys) * ROW * sizeof(__bf16);
  __device__ static void stage(__bf16* buf, const bf16x8 (&vd)[8], int g, int c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) st8<__bf16>(buf + (8 * g + i) * ROW + 8 * c, vd[i]);
  }
  // Transpose read: within each 16-lane group, result lane 4i+e element k is
  // element e of the 8 bytes addressed by lane i+4k.  Lane (g, s) therefore
  // addresses row (4g + s/4) [then +16], columns 16*db + 4*(s%4) .. +3, and
  // receives V[key(g, t)][16*db + s] for t = 0..7.
  __device__ static bf16x8 frag(const __bf16* buf, int db, int g, int s) {
    const __bf16* p0 = buf + (4 * g + (s >> 2)) * ROW + 16 * db + 4 * (s & 3);
    const s16x4 a = lds_read_tr(p0);
    const s16x4 b = lds_read_tr(p0 + 16 * ROW);
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  }
};

template <> struct DecV<float> {
  // Transposed [128 d][36]: slot of key kappa = 8*((kappa%16)/4) + 4*(kappa/16) + kappa%4.
  static constexpr int VS = kDecKeys + 4;
  static constexpr size_t BYTES = size_t(kHeadDim) * VS * sizeof(float);
  __device__ static void put4(float* dst, const f32x8 (&x)[8], int base, int e) {
    f32x4 y;
    y[0] = x[base + 0][e];
    y[1] = x[base + 1][e];
    y[2] = x[base + 2][e];
    y[3] = x[base + 3][e];
    *reinterpret_cast<f32x4*>(dst) = y;
  }
  __device__ static void stage(float* buf, const f32x8 (&vd)[8], int g, int c) {
    const int pos0 = 16 * (g & 1) + 4 * (g >> 1);  // keys 8g .. 8g+3
    const int pos1 = pos0 + 8;                      // keys 8g+4 .. 8g+7
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float* row = buf + (8 * c + e) * VS;
      put4(row + pos0, vd, 0, e);
      put4(row + pos1, vd, 4, e);
    }
  }
  __device__ static f32x8 frag(const float* buf, int db, int g, int s) {
    return ld8<float>(buf + (16 * db + s) * VS + 8 * g);
  }
};

template <typename T>
struct Chunk {
  v8_t<T> k[2][kHeadDim / 32];  // A operands of S^T: key 16*blk + c, d-slots 32*st + 8*g ..
  v8_t<T> v[8];                 // V rows 8*g + i, d-chunk c
  f32x4 rl[2];                  // bias of keys 16*blk + 4*g .. +3 (log2 units)
};

// The same step from MXFP8 caches: E4M3 codes with one E8M0 scale per 32
// values of D.  The score MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) takes all
// of D at once: lane (g, c) supplies bytes d = 16g .. 16g+15 and
// 64+16g .. 64+16g+15 of its key and the scale of d-block g (the operand
// layout, checked on the device: lane 16*blk + r carries the scale of row r,
// d-block blk).  V codes are dequantised to bf16 before the LDS tile.
typedef int i32x8 __attribute__((ext_vector_type(8)));
struct ChunkMX {
  i32x8 k[2];        // key 16*blk + c: d 16g .. 16g+15, then 64+16g .. 64+16g+15
  unsigned ks[2];    // E8M0 scale of that key's d-block g
  uint2 v[8];        // key 8g + i: codes of d 8c .. 8c+7
  unsigned vs[8];    // E8M0 scale of key 8g + i, d-block c/4
  f32x4 rl[2];
};

template <bool C, typename A, typename B> struct Pick { typedef A type; };
template <typename A, typename B> struct Pick<false, A, B> { typedef B type; };

// Per-workgroup reduction of the four waves' partial states (reuses the V tiles' LDS).
struct DecReduce {
  float m[kDecWaves][16];
  float l[kDecWaves][16];
  float o[kDecWaves][16][kHeadDim];
};

template <typename T>
constexpr size_t dec_static_lds() {
  return kDecWaves * DecV<T>::BYTES > sizeof(DecReduce) ? kDecWaves * DecV<T>::BYTES : sizeof(DecReduce);
}

// PAGED: the paged form (rel_attn_decode_paged): per-sequence cache lengths
// kv_len[b] (at most L), pages of page_size keys (a multiple of 32) through a
// block table, steps aligned to 32 keys so each lies in one page, and bias
// rows in distance order scaled by log2(e) only (s applied here per sequence),
// shifted per sequence so that each step's 4-key groups are aligned vectors.
// MX: MXFP8 caches (rel_attn_decode_mx); q is quantised to MXFP8 the same way
// for the score product, V is dequantised to bf16 for PV.
// BL: the bias is made in the kernel.  A workgroup whose split holds keys
// within E of the query computes s * log2(e) * r.P[:, Lb-1-j] for those keys
// and its query heads once, before its loop (16-key blocks, one MFMA chain
// per block over d_r), into a dynamic LDS region [heads][bias_ld]; its steps
// read the bias from there.  Workgroups of other splits load no bias at all
// and no pre-pass launch is needed.  Without BL the bias comes from the
// pre-pass rows in the workspace.
template <typename T, bool PAGED, bool MX = false, bool BL = false>
__global__ __launch_bounds__(kDecWaves * 64, sizeof(T) == 2 ? 2 : 1) void decode_split_kernel(DecodeArgs p) {
  static_assert(!MX || sizeof(T) == 2, "MXFP8 caches come with bf16 queries");
  using CH = typename Pick<MX, ChunkMX, Chunk<T>>::type;
  using VS = DecV<T>;
  constexpr int D = kHeadDim;
  constexpr size_t SMEM = dec_static_lds<T>();
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  extern __shared__ __attribute__((aligned(16))) float bias_lds[];  // BL: [bias_rows][bias_ld]

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;  // lane group: k-slots 8g..8g+7, accumulator rows 4g..4g+3
  const int c = lane & 15;  // query head column / A-operand row

  const int L = p.L, Hq = p.Hq, Hkv = p.Hkv, G = Hq / Hkv;

  // workgroup -> (batch, split, kv head, head group).  Its four waves take
  // interleaved 32-key steps of the split, so the workgroup streams one
  // contiguous window of the cache; neighbouring workgroups take the kv heads
  // of the same key range ([L, Hkv, D] interleaves the heads of a position).
  // Workgroup ids go round the 8 XCDs; the kv heads of one (sequence,
  // split, head group) t take ids 8 apart, so one XCD reads the whole
  // [Hkv, D] rows of its key range, each at about the same time.
  const long long x = blockIdx.x;
  const long long grp = 8LL * Hkv;
  const int kvh = (int)((x % grp) / 8);
  const long long t = (x / grp) * 8 + (x % 8);
  if (t >= (long long)p.B * p.n_split * p.n_hg) return;  // padding of the last group of 8
  const int hg = (int)(t % p.n_hg);
  long long rest = t / p.n_hg;
  // Splits in reverse order: the last split (whose workgroups also make the
  // bias) takes the lowest t of its sequence, so with an even split count
  // and one head group it runs on an even XCD; the odd XCDs of this part
  // stream a few percent slower (per-workgroup timestamps).
  const int split = p.n_split - 1 - (int)(rest % p.n_split);
  const int b = (int)(rest / p.n_split);

  // keys [ks_lo, ke) of this split; steps start at ks (= ks_lo, or ks_lo
  // rounded down to 32 keys in the paged form, the keys below ks_lo masked)
  // the first n_extra splits take extra more keys (the last split, which
  // also makes the bias, that many fewer)
  const int off = split * p.chunk + min(split, p.n_extra) * p.extra;
  const int len = p.chunk + (split < p.n_extra ? p.extra : 0);
  int Lb = L, ks_lo = p.kv_lo + off;
  float c1 = p.c1, bscale = 1.0f;
  if constexpr (PAGED) {
    Lb = min(max(p.kv_len[b], 1), min(L, p.max_pages * p.page_size));
    ks_lo = ((p.W > 0 && Lb > p.W) ? Lb - p.W : 0) + off;
    if (p.log_scale) {  // s = max(1, ln(kv_len) / ln(4096)), one per sequence
      bscale = fmaxf(1.0f, logf(float(Lb)) * (1.0f / 8.317766166719343f));
      c1 = bscale * p.alpha * 1.4426950408889634f;
    }
  }
  const int ks = PAGED ? (ks_lo & ~31) : ks_lo;
  const int ke = min(ks_lo + len, Lb);
  const bool empty = ks_lo >= Lb;  // a split past a short sequence's keys

  const int hin = hg * 16 + c;  // head within the kv group
  const bool hvalid = hin < G;
  const int h = kvh * G + (hvalid ? hin : 0);

  // BL: keys [jb, ke) carry bias; sb is the first step holding one of them
  const int jb = max(ks_lo, Lb - p.E);
  const bool has_bias = BL && p.E > 0 && jb < ke;
  const int sb = ks + ((max(jb, ks) - ks) & ~31);
  const float c2s = PAGED ? bscale * p.c2 : p.c2;

  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  // query (B operand of S^T = K Q^T): k-slot 8g+t of step st is d = 32*st + 8*g + t
  v8_t<T> qreg[D / 32];
  i32x8 qx;          // MX: the query in MXFP8, bytes as the scaled MFMA takes them
  unsigned qs = 127; // MX: E8M0 scale of d-block g of head c
  if constexpr (!MX) {
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
      qreg[st] = ld8_or_zero<T>(qg + (size_t(b) * Hq + h) * D + 32 * st + 8 * g, hvalid);
  } else {
    // every lane of head c reads the whole row, finds the four block maxima
    // and encodes its own 32 values (d 16g .. +15 and 64+16g .. +15)
    float qv[D];
#pragma unroll
    for (int v8 = 0; v8 < D / 8; ++v8) {
      const v8_t<T> x = ld8_or_zero<T>(qg + (size_t(b) * Hq + h) * D + 8 * v8, hvalid);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[8 * v8 + e] = float(x[e]);
    }
    int sh[D / kMxBlock];
#pragma unroll
    for (int blk = 0; blk < D / kMxBlock; ++blk) {
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < kMxBlock; ++e) amax = fmaxf(amax, fabsf(qv[kMxBlock * blk + e]));
      sh[blk] = mx_shared_exp(amax);
    }
    // g selects among compile-time offsets with a branch-free pick
    int shg = sh[0], lo_sh = sh[0], hi_sh = sh[2];
    if (g == 1) { shg = sh[1]; }
    if (g == 2) { shg = sh[2]; lo_sh = sh[1]; hi_sh = sh[3]; }
    if (g == 3) { shg = sh[3]; lo_sh = sh[1]; hi_sh = sh[3]; }
    qs = unsigned(shg + 127);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      if (gg != g) continue;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const int d0 = 16 * gg + 4 * w4, d1 = 64 + 16 * gg + 4 * w4;
        qx[w4] = int(e4m3_pack4(qv[d0], qv[d0 + 1], qv[d0 + 2], qv[d0 + 3], lo_sh));
        qx[4 + w4] = int(e4m3_pack4(qv[d1], qv[d1 + 1], qv[d1 + 2], qv[d1 + 3], hi_sh));
      }
    }
  }
  // bias rows (log2-scaled s * r.P, reversed): key j reads entry j - L + rl_base
  const float* rlrow = p.rl + (size_t(b) * Hq + h) * p.rl_stride;

  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = zero4();
  // Running max in log2 units.  It starts finite so exp2(x - m_run) of a masked
  // score is exactly 0 and never NaN.
  float m_run = -1e30f, l_run = 0.0f;

  T* vbuf = reinterpret_cast<T*>(smem + w * VS::BYTES);
  const size_t row_stride = size_t(Hkv) * D;
  const T* kbase = kg + (size_t(b) * L * Hkv + kvh) * D;
  const T* vbase = vg + (size_t(b) * L * Hkv + kvh) * D;
  // MX: codes (one byte per value) and scales (D / 32 bytes per row)
  typedef unsigned char u8;
  constexpr int NSC = D / kMxBlock;
  const size_t mrow = size_t(Hkv) * D, srow = size_t(Hkv) * NSC;
  const u8* kc = static_cast<const u8*>(p.k);
  const u8* vc = static_cast<const u8*>(p.v);
  const u8* ksc = static_cast<const u8*>(p.k_scale);
  const u8* vsc = static_cast<const u8*>(p.v_scale);

  // Every load of a step is unconditional, so the compiler's wait before a
  // step covers only that step's loads and later steps' stay in flight: rows
  // past the split end are clamped to its last key (masked later, weight
  // exactly 0 against finite data).
  auto fetch = [&](int j0, CH& ch) {
    // rows past the split end are clamped to its last key; in the paged form
    // the clamped rows of a step share one page: the page of min(j0, ke-1)
    const T* kb = kbase;
    const T* vb = vbase;
    int jp = 0;                   // first key of that page
    size_t r0 = size_t(b) * L;    // cache row of key jp
    if constexpr (PAGED) {
      const int jsel = max(min(j0, ke - 1), 0);
      const int pi = min(jsel / p.page_size, p.max_pages - 1);
      const int pg = min(max(p.btab[size_t(b) * p.max_pages + pi], 0), p.num_pages - 1);
      jp = pi * p.page_size;
      r0 = size_t(pg) * p.page_size;
      kb = kg + (r0 * Hkv + kvh) * D;
      vb = vg + (r0 * Hkv + kvh) * D;
    }
    if constexpr (MX) {
      // rows of sequence b (or of the page) of kv head kvh
      const u8* kcb = kc + r0 * mrow + size_t(kvh) * D;
      const u8* vcb = vc + r0 * mrow + size_t(kvh) * D;
      const u8* ksb = ksc + r0 * srow + size_t(kvh) * NSC;
      const u8* vsb = vsc + r0 * srow + size_t(kvh) * NSC;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int j = min(j0 + 16 * blk + c, ke - 1) - jp;
        const uint4 lo = *reinterpret_cast<const uint4*>(kcb + size_t(j) * mrow + 16 * g);
        const uint4 hi = *reinterpret_cast<const uint4*>(kcb + size_t(j) * mrow + 64 + 16 * g);
        ch.k[blk] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        ch.ks[blk] = ksb[size_t(j) * srow + g];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = min(j0 + 8 * g + i, ke - 1) - jp;
        ch.v[i] = *reinterpret_cast<const uint2*>(vcb + size_t(j) * mrow + 8 * c);
        ch.vs[i] = vsb[size_t(j) * srow + (c >> 2)];
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int j = min(j0 + 16 * blk + c, ke - 1);
        const T* src = kb + size_t(j - jp) * row_stride + 8 * g;
#pragma unroll
        for (int st = 0; st < D / 32; ++st) ch.k[blk][st] = ld8<T>(src + 32 * st);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = min(j0 + 8 * g + i, ke - 1);
        ch.v[i] = ld8<T>(vb + size_t(j - jp) * row_stride + 8 * c);
      }
    }
    if constexpr (BL) {
      // bias from LDS in process()
    } else if constexpr (PAGED) {
      // Bias of key j at distance d = Lb-1-j: the row is in distance order
      // from entry sh = (4 - Lb % 4) % 4 on (zeros from distance E to the row's
      // end), so keys j0+16*blk+4g .. +3 are the four entries from
      // Lb-4-(j0+16*blk+4g)+sh, 16-byte aligned, in reverse order.  Clamping
      // keeps the read inside the row: a group clamped to the end is at
      // distances >= E (zeros); one clamped to the start holds only keys past
      // Lb-1, which are masked.
      if (p.E > 0) {
        const int sh = (4 - (Lb & 3)) & 3;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int idx = min(max(Lb - 4 - (j0 + 16 * blk + 4 * g) + sh, 0), p.rl_stride - 4);
          const f32x4 t = *reinterpret_cast<const f32x4*>(rlrow + idx);
          ch.rl[blk] = f32x4{t[3], t[2], t[1], t[0]};
        }
      } else {
        ch.rl[0] = zero4();
        ch.rl[1] = zero4();
      }
    } else {
      // Bias of keys j0+16*blk+4g .. +3: entries j - L + rl_base.  Clamping
      // keeps the read inside the row; a clamped key is at distance >= E, whose
      // entry (like every entry beyond the extent) holds exactly 0.
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int idx = min(max(j0 + 16 * blk + 4 * g - L + p.rl_base, 0), p.rl_stride - 4);
        ch.rl[blk] = *reinterpret_cast<const f32x4*>(rlrow + idx);
      }
    }
  };

  auto process = [&](int j0, CH& ch) {
    f32x4 x[2];
    if constexpr (MX) {
      // V codes -> bf16 (exact: a 4-bit significand times a power of two)
      v8_t<T> vd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sc = e8m0_float(ch.vs[i]);
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ch.v[i].x, sc, false);
        const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ch.v[i].x, sc, true);
        const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ch.v[i].y, sc, false);
        const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ch.v[i].y, sc, true);
        vd[i] = v8_t<T>{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      }
      VS::stage(vbuf, vd, g, c);
      // scores: one MXFP8 MFMA per 16 keys covers all of D
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        x[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ch.k[blk], qx, zero4(), 0, 0, 0, int(ch.ks[blk]), 0,
                                                                 int(qs));
    } else {
      VS::stage(vbuf, ch.v, g, c);
      // scores in log2 units: accumulator (blk, v) of lane (g, c) = key j0 + 16*blk + 4*g + v, head c
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        x[blk] = zero4();
#pragma unroll
        for (int st = 0; st < D / 32; ++st) mma16(ch.k[blk][st], qreg[st], x[blk]);
      }
    }
    if constexpr (BL) {
      f32x4 bb[2] = {zero4(), zero4()};
      if (has_bias && j0 >= sb) {  // steps are 32-key aligned to sb
        const float* brow = bias_lds + min(c, p.bias_rows - 1) * p.bias_ld;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          bb[blk] = *reinterpret_cast<const f32x4*>(brow + min(j0 + 16 * blk + 4 * g - sb, p.bias_cols - 4));
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) x[blk][v] = fmaf(x[blk][v], c1, bb[blk][v]);
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) x[blk][v] = fmaf(x[blk][v], c1, PAGED ? bscale * ch.rl[blk][v] : ch.rl[blk][v]);
    }
    if (j0 + kDecKeys > ke || (PAGED && j0 < ks_lo)) {  // ragged end (or aligned start) of the split
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = j0 + 16 * blk + 4 * g + v;
          if (j >= ke || (PAGED && j < ks_lo)) x[blk][v] = -INFINITY;
        }
    }

    // online softmax per head (lanes c, c+16, c+32, c+48); O is rescaled only
    // when some row max grows by more than 2^kLazyRescale
    float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[i][v] *= corr;
    }
    float psum = 0.0f;
    v8_t<T> pb;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = fast_exp2(x[blk][v] - m_run);
        psum += e;
        pb[4 * blk + v] = T(e);
      }
    l_run += psum;

    wave_lds_fence();
#pragma unroll
    for (int db = 0; db < D / 16; ++db) mma16(VS::frag(vbuf, db, g, c), pb, o[db]);
    wave_lds_fence();
  };

  // Wave w takes steps w, w+4, w+8, ... of the split through a ring of
  // kDecDepth buffers: a step is consumed while the next kDecDepth-1 are in
  // flight.  Splits hold a multiple of kDecSplitQuantum keys (the last split
  // may end early: its missing keys are masked), so every fetch and every
  // process below is unconditional and the waits stay partial.
  constexpr int NB = kDecDepth;
  constexpr int STRIDE = kDecWaves * kDecKeys;
  CH ring[NB];
  // steps of this split: its keys in whole ring turns (paged: up to the
  // sequence's end); none for an empty split
  const int span = ke - ks;
  int j_end = ks + min(len, (span + NB * STRIDE - 1) / (NB * STRIDE) * (NB * STRIDE));
  if constexpr (PAGED) j_end = empty ? ks : ks + min(len + 32, (span + NB * STRIDE - 1) / (NB * STRIDE) * (NB * STRIDE));
#pragma unroll
  for (int bfi = 0; bfi < NB - 1; ++bfi) fetch(ks + w * kDecKeys + bfi * STRIDE, ring[bfi]);
  if constexpr (BL) {
    if (has_bias) {
      // keys sb + 16*bi + c (A rows: P row of distance Lb-1-j, clamped into
      // [0, E) and zeroed below by the distance of each output key), heads c
      // (B columns: r of head c); accumulator v of lane (g, c) is key
      // sb + 16*bi + 4*g + v, head c, as in the score product
      // d_r is a multiple of 16: in a last half step the lane groups past
      // d_r read clamped slots against a zero r fragment
      const int nst = (p.d_r + 31) / 32;
      const T* rrow = static_cast<const T*>(p.r) + (size_t(b) * Hq + h) * p.d_r;
      const T* pcg = static_cast<const T*>(p.pc);
      v8_t<T> rf[kMaxDr / 32];
#pragma unroll
      for (int st = 0; st < kMaxDr / 32; ++st) {
        const int off = 32 * st + 8 * g;
        rf[st] = ld8_or_zero<T>(rrow + min(off, p.d_r - 8), off < p.d_r);
      }
      const int nblk = min((ke - sb + 15) / 16, p.bias_cols / 16);
      // The P rows of kBiasBatch blocks are loaded together (blocks past the
      // last are clamped to it and not stored), so a wave waits for the
      // memory once per batch rather than once per block.
      constexpr int kBiasBatch = 4;
      for (int bi0 = w; bi0 < nblk; bi0 += kBiasBatch * kDecWaves) {
        v8_t<T> pf[kBiasBatch][kMaxDr / 32];
#pragma unroll
        for (int u = 0; u < kBiasBatch; ++u) {
          const int bi = min(bi0 + u * kDecWaves, nblk - 1);
          const int d = Lb - 1 - (sb + 16 * bi + c);
          const T* prow = pcg + size_t(min(max(d, 0), p.E - 1)) * p.d_r;
#pragma unroll
          for (int st = 0; st < kMaxDr / 32; ++st) pf[u][st] = ld8<T>(prow + min(32 * st + 8 * g, p.d_r - 8));
        }
#pragma unroll
        for (int u = 0; u < kBiasBatch; ++u) {
          const int bi = bi0 + u * kDecWaves;
          f32x4 acc = zero4();
#pragma unroll
          for (int st = 0; st < kMaxDr / 32; ++st)
            if (st < nst) mma16(pf[u][st], rf[st], acc);
          f32x4 y;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int dv = Lb - 1 - (sb + 16 * bi + 4 * g + v);
            y[v] = (dv >= 0 && dv < p.E) ? acc[v] * c2s : 0.0f;
          }
          if (bi < nblk && c < p.bias_rows)
            *reinterpret_cast<f32x4*>(bias_lds + c * p.bias_ld + 16 * bi + 4 * g) = y;
        }
      }
      __syncthreads();
    }
  }
  for (int j0 = ks + w * kDecKeys; j0 < j_end; j0 += NB * STRIDE) {
#pragma unroll
    for (int bfi = 0; bfi < NB; ++bfi) {
      fetch(j0 + (bfi + NB - 1) * STRIDE, ring[(bfi + NB - 1) % NB]);
      process(j0 + bfi * STRIDE, ring[bfi]);
    }
  }

  // workgroup reduction of the four waves' (o, m, l) by log-sum-exp
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += xor_lane(l_tot, 32);
  __syncthreads();  // every wave is done with its V tile: the LDS is reused
  DecReduce* red = reinterpret_cast<DecReduce*>(smem);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(&red->o[w][c][16 * db + 4 * g]) = o[db];
  if (g == 0) {
    red->m[w][c] = m_run;
    red->l[w][c] = l_tot;
  }
  __syncthreads();
  // thread t: head t/16, output columns 8*(t%16) .. +7
  const int hc = tid >> 4;
  const int d0 = 8 * (tid & 15);
  const int hin2 = hg * 16 + hc;
  if (hin2 >= G) return;
  float M = red->m[0][hc];
#pragma unroll
  for (int i = 1; i < kDecWaves; ++i) M = fmaxf(M, red->m[i][hc]);
  float wsum_l = 0.0f;
  f32x8 acc;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) {
    const float wt = fast_exp2(red->m[i][hc] - M);
    wsum_l += wt * red->l[i][hc];
    const f32x8 oi = *reinterpret_cast<const f32x8*>(&red->o[i][hc][d0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += wt * oi[e];
  }
  const size_t n_bh = size_t(p.B) * Hq;
  const size_t bh = size_t(b) * Hq + kvh * G + hin2;
  if (p.n_split == 1) {  // the only split: normalise and write the output here
    const float inv = 1.0f / wsum_l;
    T* const out_row = static_cast<T*>(p.out) + bh * D + d0;
    st4_f32<T>(out_row, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    st4_f32<T>(out_row + 4, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (p.lse != nullptr && d0 == 0) p.lse[bh] = (M + log2f(wsum_l)) * kLn2;
    return;
  }
  float* ws_o = p.ws + (size_t(split) * n_bh + bh) * D;
  float* ws_m = p.ws + size_t(p.n_split) * n_bh * D;
  float* ws_l = ws_m + size_t(p.n_split) * n_bh;
  *reinterpret_cast<f32x8*>(ws_o + d0) = acc;
  if (d0 == 0) {
    ws_m[size_t(split) * n_bh + bh] = M;
    ws_l[size_t(split) * n_bh + bh] = wsum_l;
  }
}

// Log-sum-exp merge of the split partials.  Workgroup (bh, quarter) merges
// output columns 32*quarter .. +31 of one (batch, head): thread (sg, d4)
// covers splits sg, sg+NSG, ... and columns 4*d4 .. 4*d4+3 of the quarter.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 32;

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs p) {
  constexpr int D = kHeadDim;
  constexpr int NSG = kMergeThreads / (kMergeCols / 4);  // split groups (32)
  __shared__ float red_m[NSG];
  __shared__ float red_l[NSG];
  __shared__ f32x4 red_o[NSG][kMergeCols / 4];

  const int bh = blockIdx.x / (D / kMergeCols);
  const int col0 = (blockIdx.x % (D / kMergeCols)) * kMergeCols;
  const int tid = threadIdx.x;
  const int d4 = tid % (kMergeCols / 4);
  const int sg = tid / (kMergeCols / 4);
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

  f32x4 acc = zero4();
  float den = 0.0f;
#pragma unroll 4
  for (int s = sg; s < p.n_split; s += NSG) {
    const float wgt = fast_exp2(ws_m[size_t(s) * n_bh + bh] - M);
    const f32x4 os = *reinterpret_cast<const f32x4*>(ws_o + (size_t(s) * n_bh + bh) * D + col0 + 4 * d4);
    den += wgt * ws_l[size_t(s) * n_bh + bh];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += wgt * os[v];
  }
  red_o[sg][d4] = acc;
  if (d4 == 0) red_l[sg] = den;
  __syncthreads();
  if (sg != 0) return;
  den = red_l[0];
#pragma unroll
  for (int i = 1; i < NSG; ++i) {
    const f32x4 y = red_o[i][d4];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += y[v];
    den += red_l[i];
  }
  const float inv = 1.0f / den;
  st4_f32<T>(static_cast<T*>(p.out) + size_t(bh) * D + col0 + 4 * d4, acc[0] * inv, acc[1] * inv,
             acc[2] * inv, acc[3] * inv);
  if (p.lse != nullptr && col0 == 0 && d4 == 0) p.lse[bh] = (M + log2f(den)) * kLn2;
}

// Few splits: one thread per (sequence, head, 4 output columns) merges them.
constexpr int kMergeSmallSplits = 16;

// NS bounds n_split (2, 4, 8 or 16): each thread issues NS split loads.
template <typename T, int NS>
__global__ __launch_bounds__(256) void decode_merge_small_kernel(DecodeArgs p) {
  constexpr int D = kHeadDim;
  const size_t n_bh = size_t(p.B) * p.Hq;
  const size_t t = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_bh * (D / 4)) return;
  const size_t bh = t / (D / 4);
  const int d4 = int(t % (D / 4));
  const float* ws_o = p.ws;
  const float* ws_m = p.ws + size_t(p.n_split) * n_bh * D;
  const float* ws_l = ws_m + size_t(p.n_split) * n_bh;
  // all splits' partials are loaded first (indices clamped, splits past
  // n_split weighted by zero), then folded
  float ms[NS], ls[NS];
  f32x4 os[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const size_t sb = size_t(min(s, p.n_split - 1)) * n_bh + bh;
    ms[s] = ws_m[sb];
    ls[s] = ws_l[sb];
    os[s] = *reinterpret_cast<const f32x4*>(ws_o + sb * D + 4 * d4);
  }
  float M = ms[0];
#pragma unroll
  for (int s = 1; s < NS; ++s)
    if (s < p.n_split) M = fmaxf(M, ms[s]);
  float den = 0.0f;
  f32x4 acc = zero4();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = s < p.n_split ? fast_exp2(ms[s] - M) : 0.0f;
    den += wgt * ls[s];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += wgt * os[s][v];
  }
  const float inv = 1.0f / den;
  st4_f32<T>(static_cast<T*>(p.out) + bh * D + 4 * d4, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (p.lse != nullptr && d4 == 0) p.lse[bh] = (M + log2f(den)) * kLn2;
}

template <typename T>
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

template <typename T, bool PAGED, bool MX = false>
hipError_t launch_decode_t(const DecodeArgs& a_in, hipStream_t stream) {
  DecodeArgs a = a_in;
  const long long grid = ((long long)a.B * a.n_hg * a.n_split + 7) / 8 * 8 * a.Hkv;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // The split that holds the last E keys also makes their bias before its
  // loop.  Measured on 64 x 8K keys (bf16 and MXFP8 caches), that costs about
  // as long as streaming K and V of half as many bytes as those E rows of P
  // (every workgroup of the split reads the same rows, mostly from cache).
  // The first splits take over that many keys (rounded to whole quanta, and
  // at least one quantum stays with the last split), so the splits finish
  // together: 106.2 -> 103.7 us (bf16), 67.0 -> 65.5 us (MXFP8).
  a.extra = 0;
  a.n_extra = 0;
  if (a.E > 0 && a.n_split >= 2) {
    const int vis = (a.W > 0 && a.L > a.W) ? a.W : a.L;
    const size_t key_bytes = MX ? 2 * (kHeadDim + kHeadDim / 32) : 2 * kHeadDim * sizeof(T);
    const size_t p_bytes = size_t(a.E < a.chunk ? a.E : a.chunk) * a.d_r * sizeof(T);
    int q = (int)((p_bytes / (2 * key_bytes) + kDecSplitQuantum / 2) / kDecSplitQuantum);
    const int last = vis - (a.n_split - 1) * a.chunk;
    q = min(q, (last - 1) / kDecSplitQuantum);
    if (q > 0) {
      const int per = (q + a.n_split - 2) / (a.n_split - 1);
      a.extra = per * kDecSplitQuantum;
      a.n_extra = q / per;
    }
  }
  // Bias made in the split kernel when its LDS region leaves room for the
  // kernel's occupancy (two workgroups per CU for bf16, one for fp32): a
  // split's keys with bias span at most min(E, chunk) + 31 entries from its
  // first biased step.
  if (a.E > 0) {
    constexpr size_t kLdsPerCu = 160 * 1024;
    const size_t budget = kLdsPerCu / (sizeof(T) == 2 ? 2 : 1) - dec_static_lds<T>();
    const int span = (a.E < a.chunk + a.extra ? a.E : a.chunk + a.extra) + 31;
    const int cols = (span + 15) / 16 * 16;
    const int ld = cols + 4;
    const int G = a.Hq / a.Hkv;
    const int rows = G < 16 ? G : 16;
    const size_t bytes = size_t(rows) * ld * sizeof(float);
    if (bytes <= budget) {
      a.bias_cols = cols;
      a.bias_ld = ld;
      a.bias_rows = rows;
      hipLaunchKernelGGL((decode_split_kernel<T, PAGED, MX, true>), dim3((unsigned)grid), dim3(kDecWaves * 64),
                         (unsigned)bytes, stream, a);
      return launch_decode_merge<T>(a, stream);
    }
  }
  {
    // bias rows of every (sequence, head): s * log2(e) * r.P[:, d], stored
    // reversed so that key j finds its distance L-1-j at entry j - L + rl_base
    // (all zeros when E == 0).  Paged form: log2(e) * r.P[:, d] in distance
    // order from entry (4 - Lb % 4) % 4 of each row, zeros past E (the
    // lengths, hence s and that shift, are per sequence and known on the
    // device).
    RelLogitsArgs ra;
    ra.r = a.r;
    ra.pc = a.pc;
    ra.out = const_cast<float*>(a.rl);
    ra.n_rows = (long long)a.B * a.Hq;
    ra.d_r = a.d_r;
    ra.E = a.E;
    ra.s = PAGED ? 1.4426950408889634f : a.c2;
    ra.out_cols = a.rl_stride;
    if (PAGED) {
      ra.shift_len = a.kv_len;
      ra.shift_hq = a.Hq;
      ra.shift_lmax = a.L < a.max_pages * a.page_size ? a.L : a.max_pages * a.page_size;
    }
    ra.out_stride = a.rl_stride;
    ra.rev_base = PAGED ? 0 : a.rl_base;
    if (!PAGED || a.E > 0) {
      hipError_t e = launch_rel_logits(sizeof(T) == 2 ? 1 : 2, ra, stream);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((decode_split_kernel<T, PAGED, MX>), dim3((unsigned)grid), dim3(kDecWaves * 64), 0, stream, a);
  return launch_decode_merge<T>(a, stream);
}

// The merge launch after the split kernel (none for a single split).
template <typename T>
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  if (a.n_split <= kMergeSmallSplits) {
    const long long threads = (long long)a.B * a.Hq * (kHeadDim / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (a.n_split <= 2)
      hipLaunchKernelGGL((decode_merge_small_kernel<T, 2>), grid, dim3(256), 0, stream, a);
    else if (a.n_split <= 4)
      hipLaunchKernelGGL((decode_merge_small_kernel<T, 4>), grid, dim3(256), 0, stream, a);
    else if (a.n_split <= 8)
      hipLaunchKernelGGL((decode_merge_small_kernel<T, 8>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_small_kernel<T, kMergeSmallSplits>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_merge_kernel<T>, dim3((unsigned)(a.B * a.Hq * (kHeadDim / kMergeCols))),
                       dim3(kMergeThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int B, int L, int Hq, int Hkv, int num_splits_req, int window, int rel_extent) {
  DecodePlan pl;
  const int G = Hq / Hkv;
  pl.n_hg = (G + 15) / 16;
  pl.kv_lo = (window > 0 && L > window) ? L - window : 0;
  const int vis = L - pl.kv_lo;
  const int max_split = (vis + kDecSplitQuantum - 1) / kDecSplitQuantum;  // >= one quantum per split
  int ns;
  if (num_splits_req > 0) {
    ns = num_splits_req;
  } else {
    // Aim for ~256 workgroups (one per CU of a 256-CU part), each streaming
    // at least two quanta so its prologue latency is amortised.  Measured on
    // 64 sequences x 8192 keys: 256 workgroups (2 splits) beat 512 (4) by
    // about 3 us of ~113; counts that do not divide over the CUs (3, 6
    // splits) are slower than either.
    const long long wgs_per_split = (long long)B * Hkv * pl.n_hg;
    long long want = wgs_per_split > 0 ? (256 + wgs_per_split - 1) / wgs_per_split : 1;  // B == 0: a no-op call
    const long long cap = (vis + 2 * kDecSplitQuantum - 1) / (2 * kDecSplitQuantum);
    if (want > cap) want = cap;
    ns = (int)(want < 1 ? 1 : want);
  }
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  int chunk = (vis + ns - 1) / ns;
  chunk = (chunk + kDecSplitQuantum - 1) / kDecSplitQuantum * kDecSplitQuantum;
  ns = (vis + chunk - 1) / chunk;  // drop splits that would be empty
  if (ns < 1) ns = 1;
  pl.n_split = ns;
  pl.chunk = chunk;
  const size_t n_bh = size_t(B) * Hq;
  pl.ws_partial_bytes = (size_t(ns) * n_bh * (kHeadDim + 2) * sizeof(float) + 255) / 256 * 256;
  // Entry index of key j is j - L + rl_base (clamped to the row).
  // rl_base >= E + 31 keeps every key of a step that has bias at an index
  // >= 0, (rl_base - L + kv_lo) % 4 == 0 makes the 4-key groups 16-byte
  // aligned (steps start at kv_lo + 32n), and the row reaches rl_base + 31 so
  // a ragged last step stays inside it.
  const int base0 = rel_extent + 31;
  pl.rl_base = base0 + (((L - pl.kv_lo - base0) % 4) + 4) % 4;
  pl.rl_stride = (pl.rl_base + 31 + 3) / 4 * 4;
  pl.ws_bytes = pl.ws_partial_bytes + n_bh * size_t(pl.rl_stride) * sizeof(float);
  return pl;
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_decode_t<__bf16, false>(a, stream);
  return launch_decode_t<float, false>(a, stream);
}

hipError_t launch_decode_paged(int dtype, const DecodeArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_decode_t<__bf16, true>(a, stream);
  return launch_decode_t<float, true>(a, stream);
}

hipError_t launch_decode_mx(const DecodeArgs& a, hipStream_t stream) {
  if (a.btab != nullptr) return launch_decode_t<__bf16, true, true>(a, stream);
  return launch_decode_t<__bf16, false, true>(a, stream);
}

}  // namespace relattn
