// av_validate.hip — device-side check of the packing arrays (cu_seqlens), the
// precondition the kernels rely on but the host cannot see: cu[0] = 0,
// non-decreasing, cu[num_seqs] = total, and no sequence longer than the
// max_seqlen the call passes (the grids, the 32-bit row offsets and the
// range-checked copies are all sized from those host values).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_launch.h"

namespace av {

// One workgroup; the result is a bit mask (see kSeqlenBits), 0 when valid.
__global__ __launch_bounds__(256) void validate_seqlens_kernel(const int32_t* __restrict__ cu_q,
                                                               const int32_t* __restrict__ cu_k, int num_seqs,
                                                               int64_t total_q, int64_t total_k, int max_q, int max_k,
                                                               int32_t* __restrict__ result) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  if (threadIdx.x == 0) {
    if (cu_q[0] != 0) f |= kSeqlenBadStart;
    if (cu_k[0] != 0) f |= kSeqlenBadStart;
    if ((int64_t)cu_q[num_seqs] != total_q) f |= kSeqlenBadTotal;
    if ((int64_t)cu_k[num_seqs] != total_k) f |= kSeqlenBadTotal;
  }
  for (int b = threadIdx.x; b < num_seqs; b += blockDim.x) {
    const int lq = cu_q[b + 1] - cu_q[b];
    const int lk = cu_k[b + 1] - cu_k[b];
    if (lq < 0 || lk < 0) f |= kSeqlenDecreasing;
    if (lq > max_q || lk > max_k) f |= kSeqlenOverMax;
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) result[0] = flags;
}

hipError_t launch_validate_seqlens(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int64_t total_q,
                                   int64_t total_k, int max_q, int max_k, int32_t* result, void* stream) {
  hipLaunchKernelGGL(validate_seqlens_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, cu_q, cu_k, num_seqs,
                     total_q, total_k, max_q, max_k, result);
  return hipGetLastError();
}

}  // namespace av
