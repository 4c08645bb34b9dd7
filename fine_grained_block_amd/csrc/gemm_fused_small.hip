// gemm_fused_small.hip — launches of the fused-quantization decode GEMM for M <= 8
// (gemm_decode_fused_quant_small_kernel: only the real activation rows are quantized, spread
// over the whole wave).  Same K split as the two-launch path's M <= 16 kernels.
#include "gemm_decode_kernels.hpp"

namespace fgb {

namespace {

template <int WK, int MQ>
void launch_small(const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N / 16)), block(64 * WK);
  if (a.s_w_fmt == 0) {
    if (a.y_dtype == 0)
      hipLaunchKernelGGL((gemm_decode_fused_quant_small_kernel<WK, MQ, 3, 0, 0>), grid, block, 0, stream, a, x, ldx);
    else
      hipLaunchKernelGGL((gemm_decode_fused_quant_small_kernel<WK, MQ, 3, 0, 1>), grid, block, 0, stream, a, x, ldx);
  } else {
    if (a.y_dtype == 0)
      hipLaunchKernelGGL((gemm_decode_fused_quant_small_kernel<WK, MQ, 3, 1, 0>), grid, block, 0, stream, a, x, ldx);
    else
      hipLaunchKernelGGL((gemm_decode_fused_quant_small_kernel<WK, MQ, 3, 1, 1>), grid, block, 0, stream, a, x, ldx);
  }
}

template <int MQ>
void launch_small_wk(int wk, const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  if (wk == 1) launch_small<1, MQ>(a, x, ldx, stream);
  else if (wk == 2) launch_small<2, MQ>(a, x, ldx, stream);
  else if (wk == 4) launch_small<4, MQ>(a, x, ldx, stream);
  else launch_small<8, MQ>(a, x, ldx, stream);
}

}  // namespace

hipError_t launch_gemm_decode_fused_small(const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  const int wk = decode_small_waves(a.N, a.K);
  if (a.M <= 1) launch_small_wk<1>(wk, a, x, ldx, stream);
  else if (a.M <= 2) launch_small_wk<2>(wk, a, x, ldx, stream);
  else if (a.M <= 4) launch_small_wk<4>(wk, a, x, ldx, stream);
  else launch_small_wk<8>(wk, a, x, ldx, stream);
  return hipGetLastError();
}

}  // namespace fgb
