// A plain streaming read of device memory: the yardstick that bench.py's
// --hbm-ceiling run sets beside the decode kernels' HBM fractions.  Not part
// of the relative-attention ABI; built into its own library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

// Each thread reads 16-byte vectors in a grid-stride loop, four loads in
// flight, and folds them into one word it writes at the end (so the reads
// cannot be dropped).  sink holds one word per thread of the grid.
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

}  // namespace

extern "C" {

// Threads the probe launches (the sink must hold this many 32-bit words).
size_t hbm_probe_threads(int blocks) { return size_t(blocks) * 256; }

// Reads the `bytes` bytes at src (device memory, 16-byte aligned, bytes a
// multiple of 16) with `blocks` workgroups of 256 threads on `stream`.
// Returns 0, -1 for bad arguments, -4 for a failed launch.
int hbm_read_probe(const void* src, size_t bytes, int blocks, unsigned* sink, void* stream) {
  if (src == nullptr || sink == nullptr || blocks <= 0 || (bytes & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
