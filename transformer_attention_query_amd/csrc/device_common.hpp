// Device helpers for the gfx950 kernels: operand vectors, MFMA wrappers,
// conversions and wave-level exchange.
//
// MFMA lane layouts used throughout (wave of 64 lanes; l = lane id):
//   32x32 tiles (v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x2_f32):
//     A[i][k]: lane l supplies row i = l%32, k-slots 8*(l/32) .. +7
//     B[k][j]: lane l supplies column j = l%32, k-slots 8*(l/32) .. +7
//     C[i][j]: lane l holds column j = l%32; accumulator v holds row
//              8*(v/4) + 4*(l/32) + v%4
//   16x16 tiles (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x4_f32):
//     A[i][k]: row i = l%16, k-slots 8*(l/16) .. +7
//     B[k][j]: column j = l%16, k-slots 8*(l/16) .. +7
//     C[i][j]: column j = l%16; accumulator v holds row 4*(l/16) + v
// A contraction only needs A and B to agree on which k each slot carries, so
// the fp32 path feeds element m of each lane's 8-vector to the m-th of eight
// K=2 (or K=4) fp32 MFMAs: the same slot -> k mapping as one bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace relattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<__bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<float> { typedef f32x8 v8; typedef f32x4 v4; };

template <typename T> using v8_t = typename Vec<T>::v8;
template <typename T> using v4_t = typename Vec<T>::v4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- loads/stores

template <typename T>
__device__ __forceinline__ v8_t<T> ld8(const T* p) {
  return *reinterpret_cast<const v8_t<T>*>(p);
}

template <typename T>
__device__ __forceinline__ void st8(T* p, const v8_t<T>& x) {
  *reinterpret_cast<v8_t<T>*>(p) = x;
}

template <typename T>
__device__ __forceinline__ v8_t<T> zero8() {
  v8_t<T> z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = T(0.0f);
  return z;
}

template <typename T>
__device__ __forceinline__ v8_t<T> ld8_or_zero(const T* p, bool ok) {
  return ok ? ld8<T>(p) : zero8<T>();
}

template <typename T>
__device__ __forceinline__ void st4_f32(T* p, float a, float b, float c, float d) {
  v4_t<T> x;
  x[0] = T(a);
  x[1] = T(b);
  x[2] = T(c);
  x[3] = T(d);
  *reinterpret_cast<v4_t<T>*>(p) = x;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ void mma32(const bf16x8& a, const bf16x8& b, f32x16& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(const f32x8& a, const f32x8& b, f32x16& c) {
#pragma unroll
  for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[m], c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(const bf16x8& a, const bf16x8& b, f32x4& c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(const f32x8& a, const f32x8& b, f32x4& c) {
#pragma unroll
  for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}
__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.0f;
  return z;
}

// ---------------------------------------------------------------- math

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- wave exchange

// Value of lane (l ^ mask) for mask in {16, 32}: a cross-lane read through
// ds_bpermute (no LDS storage used).
__device__ __forceinline__ float xor_lane(float x, int mask) {
  int l = __lane_id();
  int src = (l ^ mask) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
}

// Reductions over the lane pair (l, l ^ 32) with v_permlane32_swap, which
// exchanges the upper half of its first operand with the lower half of its
// second: with x in both, the two results hold x and x of the partner lane
// (in either order), so their max / sum is the pair's on every lane.
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (LDS executes one wave's operations in order; this keeps the compiler
// from moving the accesses across each other and waits for the writes).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace relattn
