// Measurement helpers for the benchmark; not part of the attention library's C ABI.
// Stream read: the achievable HBM read bandwidth on this device, measured with the same
// kind of loads the decode kernel issues (16 bytes per lane, fully coalesced).
// Copy: a known number of bytes read and written once, the reference that scales the
// hardware byte counters (FETCH_SIZE, WRITE_SIZE) to bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // data-dependent store keeps every load live
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device memory `buf` once.  Returns 0 on success.
extern "C" int tq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || blocks <= 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)buf,
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copies `bytes` (a multiple of 16) from `src` to `dst` (device, not overlapping).  Returns 0
// on success.
extern "C" int tq_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes % 16 != 0 || blocks <= 0) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
