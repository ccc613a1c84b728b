// Dense relative logits for gfx950 (page "SGLang and Miles Add Day-0 Support
// for Inkling", section "Attention with Relative Positional Embedding", eq.
// for rel_logits; the SGLang section "Relative Logits Optimization" runs this
// projection as its own step on a second stream):
//   out[row, d] = s * sum_c r[row, c] * P_cols[d, c],   row = (token, head)
// A plain MFMA GEMM [n_rows x d_r] x [d_r x E] with fp32 output.  Both
// operands are contiguous along the contraction, so lanes load their
// 16-byte MFMA fragments straight from global memory (P_cols is small and
// stays in L2); the fp32 output dominates the traffic.
#include "device_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

constexpr int kRlWaves = 4;
constexpr int kRlRows = 32;             // rows per workgroup
constexpr int kRlCols = 32 * kRlWaves;  // output columns per workgroup (32 per wave)

template <typename T>
__global__ __launch_bounds__(kRlWaves * 64) void rel_logits_kernel(RelLogitsArgs p) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int a = lane & 31;
  const int d_r = p.d_r, E = p.E;
  const int nk = d_r / 16;

  const long long row0 = (long long)blockIdx.x * kRlRows;
  const int col = blockIdx.y * kRlCols + 32 * w + a;  // this lane's output column (B-operand column)
  const T* rg = static_cast<const T*>(p.r);
  const T* pcg = static_cast<const T*>(p.pc);

  const long long arow = row0 + a;
  const bool aok = arow < p.n_rows && E > 0;
  const int d = p.rev_base > 0 ? p.rev_base - 1 - col : col;
  const bool bok = d >= 0 && d < E;
  f32x16 acc = zero16();
  if (E > 0) {  // with E == 0 (decode without bias) r and P may be NULL: zeros, no loads
    // every operand load is issued first, from clamped addresses inside r
    // and P, and zeroed where it falls outside them or past d_r only when used
    const T* arow_p = rg + (aok ? arow : 0) * d_r + 8 * h2;
    const T* prow = pcg + size_t(bok ? d : 0) * d_r + 8 * h2;
    v8_t<T> av[kMaxDr / 16], bv[kMaxDr / 16];
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) {
      const int kc = min(kk, nk - 1) * 16;
      av[kk] = ld8<T>(arow_p + kc);
      bv[kk] = ld8<T>(prow + kc);
    }
#pragma unroll
    for (int kk = 0; kk < kMaxDr / 16; ++kk) {
      const bool ok = kk < nk;
      mma32((aok && ok) ? av[kk] : zero8<T>(), (bok && ok) ? bv[kk] : zero8<T>(), acc);
    }
  }
  // accumulator v of lane (h2, a): row 8*(v/4) + 4*h2 + v%4, column a
  if (col < p.out_cols) {
    // Per-row shift: rows 4k .. 4k+3 belong to one sequence when shift_hq is
    // a multiple of 4, so a lane looks its shift up once per group of four.
    const bool grouped = p.shift_hq % 4 == 0;
    auto shift_of = [&](long long row) {
      if (p.shift_len == nullptr) return 0;
      const long long rr = min(row, p.n_rows - 1);
      return (4 - (min(max(p.shift_len[rr / p.shift_hq], 1), p.shift_lmax) & 3)) & 3;
    };
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const long long rg = row0 + 8 * g4 + 4 * h2;
      const int sh_g = grouped ? shift_of(rg) : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long long row = rg + e;
        if (row < p.n_rows) {
          const int sh = grouped ? sh_g : shift_of(row);
          if (col + sh < p.out_stride) p.out[row * p.out_stride + col + sh] = acc[4 * g4 + e] * p.s;
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_rel_logits_t(const RelLogitsArgs& a, hipStream_t stream) {
  const long long gx = (a.n_rows + kRlRows - 1) / kRlRows;
  const int gy = (a.out_cols + kRlCols - 1) / kRlCols;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rel_logits_kernel<T>, dim3((unsigned)gx, (unsigned)gy), dim3(kRlWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rel_logits(int dtype, const RelLogitsArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_rel_logits_t<__bf16>(a, stream);
  return launch_rel_logits_t<float>(a, stream);
}

}  // namespace relattn
