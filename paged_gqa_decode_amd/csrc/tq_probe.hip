// HBM streaming probes (read-only and copy) for measuring achievable bandwidth
// and calibrating byte counters; see include/tq_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // 8 independent non-temporal loads in flight per thread per iteration
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4* __restrict__ dst,
                                                         const u32x4* __restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int32_t tq_probe_read(const void* src, size_t n_bytes, uint32_t* sink,
                                 int32_t num_workgroups, void* stream) {
  if (!src || !sink || (n_bytes & 15) || ((uintptr_t)src & 15) || num_workgroups < 1 ||
      num_workgroups > 65536)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3(num_workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n_bytes / 16,
                     sink);
  return (int32_t)hipGetLastError();
}

extern "C" int32_t tq_probe_copy(void* dst, const void* src, size_t n_bytes, int32_t num_workgroups,
                                 void* stream) {
  if (!src || !dst || (n_bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) ||
      num_workgroups < 1 || num_workgroups > 65536)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(num_workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n_bytes / 16);
  return (int32_t)hipGetLastError();
}
