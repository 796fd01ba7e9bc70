// probe.hip -- a plain streaming read, the ceiling a bandwidth-bound kernel of
// a given size can reach on this device (measurement aid, not on the decode
// path).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace tq {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads per thread, all in flight together

// Each thread reads kProbeUnroll 16-byte words, kProbeThreads words apart, and
// folds them; the fold is stored only if it equals a constant no input of the
// measurement produces, so the loads cannot be dropped but nothing is written.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const uint4* __restrict__ p, long long n16, uint32_t* __restrict__ sink) {
  const long long base = (long long)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x;
  uint4 v[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) {
    const long long i = base + (long long)u * kProbeThreads;
    v[u] = i < n16 ? p[i] : uint4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// The second design: a resident grid, one 1024-thread workgroup per CU, each
// thread looping over its share with kResidentUnroll 16-byte loads in flight
// per pass (128 KB per CU), so that workgroup launch and drain happen once
// rather than once per 32 KB.
constexpr int kResidentThreads = 1024;
constexpr int kResidentUnroll = 8;

__global__ __launch_bounds__(kResidentThreads) void stream_read_resident_kernel(
    const uint4* __restrict__ p, long long n16, uint32_t* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * kResidentThreads;
  uint32_t acc = 0;
  for (long long i0 = (long long)blockIdx.x * kResidentThreads + threadIdx.x; i0 < n16;
       i0 += stride * kResidentUnroll) {
    uint4 v[kResidentUnroll];
#pragma unroll
    for (int u = 0; u < kResidentUnroll; ++u) {
      const long long i = i0 + (long long)u * stride;
      v[u] = i < n16 ? p[i] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kResidentUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read_resident(const void* buf, size_t bytes, uint32_t* sink,
                                       hipStream_t stream) {
  const long long n16 = (long long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // no more workgroups than there are 1024-word slices
  const long long slices = (n16 + kResidentThreads - 1) / kResidentThreads;
  const long long blocks = slices < cus ? slices : cus;
  hipLaunchKernelGGL(stream_read_resident_kernel, dim3((unsigned)blocks), dim3(kResidentThreads),
                     0, stream, (const uint4*)buf, n16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const long long n16 = (long long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const long long per_block = (long long)kProbeThreads * kProbeUnroll;
  const long long blocks = (n16 + per_block - 1) / per_block;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     (const uint4*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace tq
