// Read-rate probe: a plain one-pass stream over device memory, the yardstick for the
// HBM-bound kernels of the decode step. It reads with the load width and cache policy of the
// page-bound kernel (16-byte non-temporal loads, every load of a thread issued before any is
// used) and does the least work that keeps the loads alive: a per-workgroup fp32 sum.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "hhr.h"
#include "hhr_launch.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;                                  // 16-byte loads per thread
constexpr size_t kProbeBlockBytes = size_t(16) * kProbeLoads * kProbeThreads;   // 32 KiB

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Workgroup i reads the 16-byte elements [i * 2048, (i + 1) * 2048) of the n4 at x (thread t
// takes t, t + 256, ...: each load instruction of a wave covers 1 KiB contiguously) and writes
// the fp32 sum of the floats it read to partial[i]. Elements past n4 are not read.
__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const f32x4v* __restrict__ x, size_t n4, float* __restrict__ partial) {
  const size_t base = size_t(blockIdx.x) * (kProbeLoads * kProbeThreads) + threadIdx.x;
  f32x4v v[kProbeLoads];
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u) {
    const size_t i = base + size_t(u) * kProbeThreads;
    v[u] = __builtin_nontemporal_load(x + (i < n4 ? i : n4 - 1));
  }
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < kProbeLoads; ++u)
    if (base + size_t(u) * kProbeThreads < n4) sum += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  __shared__ float ws[kProbeThreads / 64];
  if (threadIdx.x % 64 == 0) ws[threadIdx.x / 64] = sum;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

}  // namespace

extern "C" {

size_t hhr_read_probe_blocks(size_t bytes) {
  return (bytes + kProbeBlockBytes - 1) / kProbeBlockBytes;
}

hhr_status hhr_read_probe(const void* src, size_t bytes, float* partial, hhr_stream_t stream) {
  if (!src || !partial || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return HHR_ERR_INVALID_ARG;
  const size_t blocks = hhr_read_probe_blocks(bytes);
  if (blocks > 0x7FFFFFFFull) return HHR_ERR_CAPACITY;
  const hipError_t e = hhr::launch_kernel("read_probe_kernel", 
      read_probe_kernel, dim3(unsigned(blocks)), dim3(kProbeThreads),
      reinterpret_cast<hipStream_t>(stream), hhr::KernelTimer{nullptr, nullptr},
      static_cast<const f32x4v*>(src), bytes / 16, partial);
  return e == hipSuccess ? HHR_OK : HHR_ERR_HIP;
}

}  // extern "C"
