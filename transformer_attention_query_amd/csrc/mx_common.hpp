// MXFP8 helpers for the gfx950 kernels: OCP MX blocks of 32 E4M3 elements
// sharing one E8M0 scale (the K/V storage of page "SGLang and Miles Add
// Day-0 Support for Inkling", section "Relative Logits Optimization",
// paragraph "MXFP8 Support").
//
//   E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
//         holds the subnormals m * 2^-9; no infinities; largest value 448.
//   E8M0: a byte e standing for 2^(e - 127).
//   A block's shared exponent is floor(log2(max |x|)) - 8 (8: the exponent of
//   the largest E4M3 normal), clamped to [-127, 127] (0 for an all-zero
//   block); each element is x * 2^-shared rounded to nearest, ties to even,
//   magnitudes beyond 448 clamped to 448.  Scaling by a power of two is exact,
//   so the only rounding is the one to E4M3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace relattn {

constexpr int kMxBlock = 32;

// E4M3 byte of the finite float v.
__device__ __forceinline__ unsigned e4m3_encode(float v) {
  const unsigned bits = __float_as_uint(v);
  const unsigned sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  unsigned code;
  if (a >= 0.015625f) {  // 2^-6: an E4M3 normal
    // keep 3 mantissa bits, rounding at bit 20 to nearest, ties to even; a
    // carry moves into the exponent by itself
    const unsigned ab = __float_as_uint(a);
    const unsigned t = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;  // exponent(8) : mantissa(3)
    const int c = int(t) - (120 << 3);                               // rebias 127 -> 7
    code = c > 0x7E ? 0x7Eu : unsigned(c);
  } else {
    code = unsigned(__builtin_rintf(a * 512.0f));  // subnormal quantum 2^-9, ties to even
  }
  return sign | code;
}

// Shared exponent of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;  // amax = m * 2^(e+9), m in [0.5, 1)
  return min(max(e, -127), 127);
}

// Four values scaled by 2^-shared, as four E4M3 bytes in one dword (element 0
// in the low byte).
__device__ __forceinline__ unsigned e4m3_pack4(float a, float b, float c, float d, int shared) {
  return e4m3_encode(__builtin_amdgcn_ldexpf(a, -shared)) | (e4m3_encode(__builtin_amdgcn_ldexpf(b, -shared)) << 8) |
         (e4m3_encode(__builtin_amdgcn_ldexpf(c, -shared)) << 16) |
         (e4m3_encode(__builtin_amdgcn_ldexpf(d, -shared)) << 24);
}

// Largest value over the quad of lanes 4j .. 4j+3 (the four lanes that hold
// one 32-value block when a row of 128 is spread over 16 lanes).
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));  // quad_perm 1,0,3,2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));  // quad_perm 2,3,0,1
  return x;
}

// 2^(e - 127) as a float for the scaled conversions (which use only the
// exponent of their scale operand); e in [1, 254].
__device__ __forceinline__ float e8m0_float(unsigned e) { return __uint_as_float(e << 23); }

}  // namespace relattn
