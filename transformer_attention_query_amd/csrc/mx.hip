// MXFP8 quantisation of rows of D = 128 values (gfx950): E4M3 codes and one
// E8M0 scale per 32 values (see mx_common.hpp for the format and the
// rounding).  Sixteen lanes own a row, eight values each; the four lanes of a
// 32-value block take its maximum magnitude with two DPP quad exchanges.
// Used to fill MXFP8 caches from existing bf16 / fp32 rows (the prologue
// quantises new rows itself).
#include "device_common.hpp"
#include "mx_common.hpp"
#include "relattn_internal.hpp"

namespace relattn {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T* __restrict__ x, unsigned char* __restrict__ codes,
                                                          unsigned char* __restrict__ scales, long long n_rows) {
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= n_rows) return;  // whole 16-lane groups
  const int l16 = threadIdx.x & 15;
  const v8_t<T> v = ld8<T>(x + row * kHeadDim + 8 * l16);
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = float(v[e]);
    amax = fmaxf(amax, fabsf(f[e]));
  }
  const int sh = mx_shared_exp(quad_max(amax));
  uint2 out;
  out.x = e4m3_pack4(f[0], f[1], f[2], f[3], sh);
  out.y = e4m3_pack4(f[4], f[5], f[6], f[7], sh);
  *reinterpret_cast<uint2*>(codes + row * kHeadDim + 8 * l16) = out;
  if ((l16 & 3) == 0) scales[row * (kHeadDim / kMxBlock) + (l16 >> 2)] = (unsigned char)(sh + 127);
}

template <typename T>
hipError_t launch_t(const void* x, void* codes, void* scales, long long n_rows, hipStream_t stream) {
  const long long grid = (n_rows + 15) / 16;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_quantize_kernel<T>, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const T*>(x),
                     static_cast<unsigned char*>(codes), static_cast<unsigned char*>(scales), n_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize(int dtype, const void* x, void* codes, void* scales, long long n_rows,
                              hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  if (dtype == 1) return launch_t<__bf16>(x, codes, scales, n_rows, stream);
  return launch_t<float>(x, codes, scales, n_rows, stream);
}

}  // namespace relattn
