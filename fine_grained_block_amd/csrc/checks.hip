// checks.hip — device-side check of the grouped GEMM's expert offsets (a debugging aid: the
// grouped kernels take the offsets as a precondition, since checking them before a launch would
// need a device synchronization).  The layout is rows sorted by expert, expert e owning rows
// offsets[e] .. offsets[e+1]-1 (Transformers "Fine-grained FP8", the expert matmuls).
#include "internal.h"

namespace fgb {
namespace {

// result = 0 when offsets[0] == 0, offsets is nondecreasing and offsets[E] == total_M; otherwise
// 1 + the first index i in 0..E whose entry breaks that (i = 0: nonzero start; i > 0:
// offsets[i] < offsets[i-1], or i = E: offsets[E] != total_M).
__global__ __launch_bounds__(256) void check_offsets_kernel(const int32_t* __restrict__ off, int E, int64_t total_M,
                                                            int32_t* __restrict__ result) {
  __shared__ int first;
  if (threadIdx.x == 0) first = 0x7fffffff;
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += blockDim.x) {
    const int32_t v = off[i];
    bool bad = false;
    if (i == 0) bad = v != 0;
    else bad = v < off[i - 1];
    if (i == E) bad = bad || (int64_t)v != total_M;
    if (bad) atomicMin(&first, i);
  }
  __syncthreads();
  if (threadIdx.x == 0) result[0] = first == 0x7fffffff ? 0 : first + 1;
}

}  // namespace

hipError_t launch_check_offsets(const int32_t* offsets, int32_t E, int64_t total_M, int32_t* result,
                                hipStream_t stream) {
  hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(256), 0, stream, offsets, (int)E, total_M, result);
  return hipGetLastError();
}

}  // namespace fgb
