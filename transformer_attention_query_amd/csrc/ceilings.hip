// Yardsticks that bench.py sets beside the kernels' fractions of the
// published peaks: what plain code of each kind reaches on this GPU.
//   hbm_read_kernel   a streaming read of device memory (--hbm-ceiling)
//   mfma_kernel       back-to-back bf16 v_mfma_f32_32x32x16 (--ceilings)
//   exp_kernel        independent v_exp_f32 chains (--ceilings)
//   lds_kernel        16-byte LDS reads, no bank conflicts (--ceilings)
//   clock_kernel      the shader clock against the 100 MHz real-time counter
// Not part of the relative-attention ABI; built into its own library.  Every
// kernel writes one word per thread to a sink the caller sizes with
// ceiling_threads(), so the work cannot be dropped.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each thread reads 16-byte vectors in a grid-stride loop, four loads in
// flight, and folds them into one word it writes at the end.
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ src, size_t n_vec,
                                                      unsigned* __restrict__ sink) {
  const size_t tid = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  unsigned acc = 0;
  size_t i = tid;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[tid] = acc;
}

// Four independent accumulators per wave, so consecutive MFMAs never wait
// for each other's result: iters x 4 MFMAs of 32x32x16 (32768 flops each).
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float(lane + i) * (1.0f / 64.0f));
    b[i] = __bf16(float(i - lane) * (1.0f / 64.0f));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains per thread: iters x 8 v_exp_f32 (plus one
// multiply each, which keeps the values in range).
__global__ __launch_bounds__(256) void exp_kernel(int iters, float* __restrict__ sink) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = float(threadIdx.x & 7) * 0.01f + 0.1f * float(k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(x[k] * -0.5f);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Each wave reads 16 bytes per lane per instruction from a 16 KB LDS buffer,
// four reads per iteration.  ROWS = false: lane l at byte 16 l plus a
// per-iteration offset (consecutive lanes, consecutive bytes).  ROWS = true:
// the pattern of an MFMA fragment read from a tile of 304-byte rows (lane
// (a, h) at byte 304 a + 16 h, the four reads 32 bytes apart).
template <bool ROWS>
__global__ __launch_bounds__(256) void lds_kernel(int iters, unsigned* __restrict__ sink) {
  __shared__ u32x4 buf[1024];
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) {
    const unsigned u = unsigned(i);
    buf[i] = u32x4{u, u * 3u, u * 5u, u * 7u};
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int frag = 19 * (lane & 31) + (lane >> 5);  // 16-byte unit of lane (a, h) in 304-byte rows
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    const int base = (it * 256) & 1023;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = ROWS ? frag + 2 * ((it * 4 + k) & 7) : (base + 64 * k + lane) & 1023;
      // volatile, in the LDS address space: one ds_read_b128 per read, none hoisted
      const u32x4 v = *((volatile __attribute__((address_space(3))) u32x4*)(
          (__attribute__((address_space(3))) void*)&buf[idx]));
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// The shader clock (s_memtime) and the real-time counter (s_memrealtime,
// 100 MHz) read at the start and the end of a VALU loop; thread 0 of each
// workgroup writes both differences.
__global__ __launch_bounds__(256) void clock_kernel(int iters, unsigned long long* __restrict__ out,
                                                   float* __restrict__ sink) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = float(threadIdx.x) * 1e-3f;
  for (int it = 0; it < iters; ++it) x = fmaf(x, 0.999f, 1e-3f);
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = x;
  __syncthreads();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * size_t(blockIdx.x)] = c1 - c0;
    out[2 * size_t(blockIdx.x) + 1] = r1 - r0;
  }
}

hipError_t launched() { return hipGetLastError(); }

}  // namespace

extern "C" {

// Threads a probe launches with `blocks` workgroups of 256 (the sink must
// hold this many 32-bit words).
size_t ceiling_threads(int blocks) { return size_t(blocks) * 256; }

// Reads the `bytes` bytes at src (device memory, 16-byte aligned, bytes a
// multiple of 16) with `blocks` workgroups of 256 threads on `stream`.
// Returns 0, -1 for bad arguments, -4 for a failed launch.
int hbm_read_probe(const void* src, size_t bytes, int blocks, unsigned* sink, void* stream) {
  if (src == nullptr || sink == nullptr || blocks <= 0 || (bytes & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return launched() == hipSuccess ? 0 : -4;
}

// kind 0: MFMA (flops = blocks x 4 waves x iters x 4 x 32768), 1: exp
// (blocks x 256 x iters x 8 exponentials), 2: LDS, consecutive bytes, 3: LDS,
// fragment pattern (both blocks x 256 x iters x 4 x 16 bytes).  `blocks`
// workgroups of 256 threads; sink: ceiling_threads(blocks) words.  Returns 0,
// -1 for bad arguments, -4 for a failed launch.
int compute_probe(int kind, int blocks, int iters, void* sink, void* stream) {
  if (sink == nullptr || blocks <= 0 || iters <= 0 || kind < 0 || kind > 3) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, iters, static_cast<float*>(sink));
  else if (kind == 1)
    hipLaunchKernelGGL(exp_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, iters, static_cast<float*>(sink));
  else if (kind == 2)
    hipLaunchKernelGGL(lds_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, s, iters, static_cast<unsigned*>(sink));
  else
    hipLaunchKernelGGL(lds_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, s, iters, static_cast<unsigned*>(sink));
  return launched() == hipSuccess ? 0 : -4;
}

// out: 2 x blocks 64-bit words (shader-clock and real-time ticks of each
// workgroup); sink: ceiling_threads(blocks) words.
int clock_probe(int blocks, int iters, unsigned long long* out, float* sink, void* stream) {
  if (out == nullptr || sink == nullptr || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(clock_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     out, sink);
  return launched() == hipSuccess ? 0 : -4;
}

}  // extern "C"
