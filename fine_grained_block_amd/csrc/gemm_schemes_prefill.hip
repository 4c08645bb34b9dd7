// gemm_schemes_prefill.hip — launches of the prefill kernel (M > 64) for the scaling schemes other
// than 1x128 groups x 128x128 blocks: per-token or per-tensor activation scales with 128x128 weight
// blocks (scheme 1) or per-channel weight scales (scheme 2), E4M3 or E5M2 operands.
// (vLLM "FP8 W8A8", "Quantization process" and "Two FP8 representations"; Transformers
// "Fine-grained FP8", "DeepGEMM fast path", static activations.)
#include "gemm_prefill_kernels.hpp"

namespace fgb {

namespace {

template <typename C, int SCH, int SWF, int CODE>
void launch_sch(const GemmArgs& a, hipStream_t stream) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM), tiles_n = (int)(a.N / C::BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(C::THREADS);
  if (a.y_dtype == 0)
    hipLaunchKernelGGL((gemm_prefill_kernel<C, SWF, 0, false, SCH, CODE>), grid, block, 0, stream, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<C, SWF, 1, false, SCH, CODE>), grid, block, 0, stream, a, tiles_m, tiles_n);
}

template <typename C>
void launch_cfg_sch(const GemmArgs& a, int sch, int code, hipStream_t stream) {
  if (sch == 2) {
    if (code == 0) launch_sch<C, 2, 0, 0>(a, stream);
    else launch_sch<C, 2, 0, 1>(a, stream);
  } else if (a.s_w_fmt == 0) {
    if (code == 0) launch_sch<C, 1, 0, 0>(a, stream);
    else launch_sch<C, 1, 0, 1>(a, stream);
  } else {
    launch_sch<C, 1, 1, 0>(a, stream);  // UE8M0 block scales go with E4M3 codes
  }
}

}  // namespace

// 256 x 256 tiles where N is a multiple of 256 and K has at least 8 blocks, else 128 x 128.
hipError_t launch_gemm_scaled_prefill(const GemmArgs& a, int sch, int code, hipStream_t stream) {
  if (a.N % Big::BN == 0 && a.K >= 8 * KBYTES) launch_cfg_sch<Big>(a, sch, code, stream);
  else launch_cfg_sch<Narrow>(a, sch, code, stream);
  return hipGetLastError();
}

}  // namespace fgb
