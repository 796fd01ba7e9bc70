// cache.hip -- device side of the two-phase cache (PR #232, Design: pending
// tokens stay fp16 until a whole group is batch-compressed): moving fp16 rows
// into the pending buffer and publishing the per-sequence lengths that the
// mixed decode attention reads. Encoding itself is the encode kernel's job.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace tq {

namespace {

// blockIdx.y selects the K (0) or V (1) rows: rows [0, rows) of every head h
// go from src + h * src_head to dst + h * dst_head (16-byte words; a head's
// rows are contiguous on both sides). Workgroup (0, 0) also writes the two
// length arrays.
__global__ __launch_bounds__(256) void pending_rows_kernel(CopyRowsArgs a) {
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < a.batch; i += blockDim.x) {
      a.packed_len[i] = a.n_packed;
      a.pending_len[i] = a.n_pending;
    }
  }
  const uint4* __restrict__ src = (const uint4*)(blockIdx.y == 0 ? a.src_k : a.src_v);
  uint4* __restrict__ dst = (uint4*)(blockIdx.y == 0 ? a.dst_k : a.dst_v);
  const long long per_head = (long long)a.rows * a.row16;
  const long long total = per_head * a.heads;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long h = i / per_head, w = i - h * per_head;
    dst[h * a.dst_head + w] = src[h * a.src_head + w];
  }
}

}  // namespace

hipError_t launch_pending_rows(const CopyRowsArgs& a, hipStream_t stream) {
  const long long total = (long long)a.rows * a.row16 * a.heads;
  long long blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(pending_rows_kernel, dim3((unsigned)blocks, 2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
