// gemm_fused.hip — launches of the decode GEMM that quantizes its bf16 activations itself
// (gemm_decode_fused_quant_kernel): one launch for act_quant_group128 + w8a8_block_gemm at M <= 64.
// The K split follows the two-launch path's per-wave ring and register kernels (the same waves
// per workgroup, slices and summation order), so where that path uses them the results agree bit
// for bit.
#include "gemm_decode_kernels.hpp"

namespace fgb {

namespace {

template <int WK, int MR, int D>
void launch_fused(const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N / 16)), block(64 * WK);
  if (a.s_w_fmt == 0) {
    if (a.y_dtype == 0)
      hipLaunchKernelGGL((gemm_decode_fused_quant_kernel<WK, MR, D, 0, 0>), grid, block, 0, stream, a, x, ldx);
    else
      hipLaunchKernelGGL((gemm_decode_fused_quant_kernel<WK, MR, D, 0, 1>), grid, block, 0, stream, a, x, ldx);
  } else {
    if (a.y_dtype == 0)
      hipLaunchKernelGGL((gemm_decode_fused_quant_kernel<WK, MR, D, 1, 0>), grid, block, 0, stream, a, x, ldx);
    else
      hipLaunchKernelGGL((gemm_decode_fused_quant_kernel<WK, MR, D, 1, 1>), grid, block, 0, stream, a, x, ldx);
  }
}

template <int MR, int D>
void launch_fused_wk(int wk, const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  if (wk == 1) launch_fused<1, MR, D>(a, x, ldx, stream);
  else if (wk == 2) launch_fused<2, MR, D>(a, x, ldx, stream);
  else if (wk == 4) launch_fused<4, MR, D>(a, x, ldx, stream);
  else launch_fused<8, MR, D>(a, x, ldx, stream);
}

}  // namespace

hipError_t launch_gemm_decode_fused(const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream) {
  if (a.M <= 8) return launch_gemm_decode_fused_small(a, x, ldx, stream);
  if (a.M <= 16) {
    const int wk = decode_small_waves(a.N, a.K);
    launch_fused_wk<16, 3>(wk, a, x, ldx, stream);
  } else if (a.M <= 32) {
    launch_fused<4, 32, 3>(a, x, ldx, stream);
  } else {
    launch_fused<4, 64, 2>(a, x, ldx, stream);
  }
  return hipGetLastError();
}

}  // namespace fgb
