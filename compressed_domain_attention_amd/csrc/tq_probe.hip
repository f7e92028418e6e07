// Measurement helpers for the benchmark; not part of the attention library's C ABI.
// Stream read: the achievable HBM read bandwidth on this device.  Every workgroup streams one
// contiguous range with eight 16-byte non-temporal loads in flight per lane, the access
// pattern and cache policy of the decode kernel's streamed copies; on this chip it reads
// about 7.0 TB/s where default-policy loads reach 6.0-6.3 TB/s.
// Copy: a known number of bytes read and written once, the reference that scales the
// hardware byte counters (FETCH_SIZE, WRITE_SIZE) to bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const v4u* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  // the range of this workgroup: an equal share, the last one taking the remainder
  const size_t per = n16 / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = blockIdx.x + 1 == gridDim.x ? n16 : lo + per;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    v4u a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < hi; i += 256) {
    const v4u a = __builtin_nontemporal_load(p + i);
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
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const v4u*)buf,
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
