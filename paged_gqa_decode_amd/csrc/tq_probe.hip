// HBM streaming probes (read-only, copy, and the decode's byte pattern) for
// measuring achievable bandwidth and calibrating byte counters; see
// include/tq_probe.h.
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

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kPatChunk = 4096;  // bytes of K and of V per chunk (32 tokens x 128)

// The byte pattern of the decode's stream with no arithmetic: each wave walks
// `chunks` chunks; per chunk 4 KiB of K into registers (two 16-byte loads per
// lane per 16-token tile), 4 KiB of V and 256 B of scales into LDS by
// LDS-direct loads (16 and 4 bytes per lane, non-temporal), the next chunk
// issued once the current one is drained and read.  Workgroups of 8 waves.
__global__ __launch_bounds__(512) void probe_pattern_kernel(const uint8_t* __restrict__ k,
                                                            const uint8_t* __restrict__ v,
                                                            const float* __restrict__ sc,
                                                            int chunks, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[8][kPatChunk + 256];
  __shared__ __attribute__((aligned(16))) uint8_t sb[8][kPatChunk + 256];
  constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t gw = (size_t)blockIdx.x * 8 + wave;
  const uint8_t* kw = k + gw * (size_t)chunks * kPatChunk;
  const uint8_t* vw = v + gw * (size_t)chunks * kPatChunk;
  const float* sw = sc + gw * (size_t)chunks * 64;
  i32x4 acc = {0, 0, 0, 0};
  int lacc = 0;
  auto issue = [&](int c, uint8_t* st, i32x4* r) {
    const uint8_t* kc = kw + (size_t)c * kPatChunk;
    r[0] = *reinterpret_cast<const i32x4*>(kc + 32 * lane);
    r[1] = *reinterpret_cast<const i32x4*>(kc + 32 * lane + 16);
    r[2] = *reinterpret_cast<const i32x4*>(kc + 2048 + 32 * lane);
    r[3] = *reinterpret_cast<const i32x4*>(kc + 2048 + 32 * lane + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(vw + (size_t)c * kPatChunk + 1024 * j + 16 * lane,
                                       (lds_void*)(st + 1024 * j), 16, 0, 2);
    __builtin_amdgcn_global_load_lds(sw + (size_t)c * 64 + lane, (lds_void*)(st + kPatChunk), 4, 0, 2);
  };
  i32x4 ra[4], rb[4];
  if (chunks > 0) issue(0, sa[wave], ra);
  for (int c = 0; c < chunks; c += 2) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    lacc += *reinterpret_cast<const int*>(sa[wave] + 64 * lane) +
            *reinterpret_cast<const int*>(sa[wave] + kPatChunk + 4 * (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= ra[i];
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 >= chunks) break;
    issue(c + 1, sb[wave], rb);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    lacc += *reinterpret_cast<const int*>(sb[wave] + 64 * lane) +
            *reinterpret_cast<const int*>(sb[wave] + kPatChunk + 4 * (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= rb[i];
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < chunks) issue(c + 2, sa[wave], ra);
  }
  uint32_t x = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ lacc);
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t red[8];
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < 8; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

extern "C" int32_t tq_probe_pattern(const void* k, const void* v, const void* scales,
                                    size_t kv_bytes, size_t scale_bytes, int32_t chunks_per_wave,
                                    int32_t num_workgroups, uint32_t* sink, void* stream) {
  const size_t waves = (size_t)num_workgroups * 8;
  if (!k || !v || !scales || !sink || ((uintptr_t)k & 15) || ((uintptr_t)v & 15) ||
      ((uintptr_t)scales & 15) || num_workgroups < 1 || num_workgroups > 65536 ||
      chunks_per_wave < 1 || waves * (size_t)chunks_per_wave * kPatChunk > kv_bytes ||
      waves * (size_t)chunks_per_wave * 256 > scale_bytes)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_pattern_kernel, dim3(num_workgroups), dim3(512), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(v), static_cast<const float*>(scales),
                     chunks_per_wave, sink);
  return (int32_t)hipGetLastError();
}

// The byte pattern of the 4-bit format's stream with no arithmetic: per chunk
// 32 rows of 128 B (4 KiB, four 1 KiB LDS-direct loads) and 192 B of
// metadata (48 lanes x 4 B) into LDS, non-temporal, the next chunk issued once
// the current one is drained and read.  Workgroups of 8 waves.
constexpr int kPat4Rows = 4096, kPat4Meta = 256, kPat4MetaUsed = 192;
__global__ __launch_bounds__(512) void probe_pattern4_kernel(const uint8_t* __restrict__ rows,
                                                             const uint8_t* __restrict__ meta,
                                                             int chunks, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[8][kPat4Rows + kPat4Meta];
  __shared__ __attribute__((aligned(16))) uint8_t sb[8][kPat4Rows + kPat4Meta];
  constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t gw = (size_t)blockIdx.x * 8 + wave;
  const uint8_t* rw = rows + gw * (size_t)chunks * kPat4Rows;
  const uint8_t* mw = meta + gw * (size_t)chunks * kPat4Meta;
  int lacc = 0;
  auto issue = [&](int c, uint8_t* st) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(rw + (size_t)c * kPat4Rows + 1024 * j + 16 * lane,
                                       (lds_void*)(st + 1024 * j), 16, 0, 2);
    const int l = lane < kPat4MetaUsed / 4 ? lane : 0;
    __builtin_amdgcn_global_load_lds(mw + (size_t)c * kPat4Meta + 4 * l,
                                     (lds_void*)(st + kPat4Rows), 4, 0, 2);
  };
  if (chunks > 0) issue(0, sa[wave]);
  for (int c = 0; c < chunks; c += 2) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    lacc += *reinterpret_cast<const int*>(sa[wave] + 64 * lane) +
            *reinterpret_cast<const int*>(sa[wave] + kPat4Rows + 4 * (lane & 31));
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 >= chunks) break;
    issue(c + 1, sb[wave]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    lacc += *reinterpret_cast<const int*>(sb[wave] + 64 * lane) +
            *reinterpret_cast<const int*>(sb[wave] + kPat4Rows + 4 * (lane & 31));
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < chunks) issue(c + 2, sa[wave]);
  }
  uint32_t x = (uint32_t)lacc;
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  __shared__ uint32_t red[8];
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < 8; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

extern "C" int32_t tq_probe_pattern4(const void* rows, const void* meta, size_t rows_bytes,
                                     size_t meta_bytes, int32_t chunks_per_wave,
                                     int32_t num_workgroups, uint32_t* sink, void* stream) {
  const size_t waves = (size_t)num_workgroups * 8;
  if (!rows || !meta || !sink || ((uintptr_t)rows & 15) || ((uintptr_t)meta & 15) ||
      num_workgroups < 1 || num_workgroups > 65536 || chunks_per_wave < 1 ||
      waves * (size_t)chunks_per_wave * kPat4Rows > rows_bytes ||
      waves * (size_t)chunks_per_wave * kPat4Meta > meta_bytes)
    return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_pattern4_kernel, dim3(num_workgroups), dim3(512), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(rows),
                     static_cast<const uint8_t*>(meta), chunks_per_wave, sink);
  return (int32_t)hipGetLastError();
}

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
