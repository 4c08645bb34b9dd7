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

// The block scheme's column split (N % 256 == 0): the first big_columns() output columns as
// 256 x 256 tiles, the rest as 256 x 128 tiles, each part in its own launch (offset weight rows,
// weight scales and output columns); else 128 x 128 tiles.  Measured at the Llama-3-8B QKV shape
// 6144x4096, M = 4096 (384 tiles of 256 x 256 before, 256 + 256 split tiles now): FP8_DYNAMIC
// 107.8 -> 93.3 us, static per-tensor E5M2 112.4 -> 97.7 us.
hipError_t launch_gemm_scaled_prefill(const GemmArgs& a, int sch, int code, hipStream_t stream) {
  if (a.N % Big::BN != 0 || a.N % Half::BN != 0) {
    launch_cfg_sch<Narrow>(a, sch, code, stream);
    return hipGetLastError();
  }
  const int64_t n_big = big_columns(a.M, a.N, a.K);
  if (n_big > 0) {
    GemmArgs b = a;
    b.N = n_big;
    launch_cfg_sch<Big>(b, sch, code, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_big == a.N) return e;
  }
  GemmArgs h = a;
  h.N = a.N - n_big;
  h.w_q = a.w_q + n_big * a.K;
  if (sch == 2)
    h.s_w = reinterpret_cast<const float*>(a.s_w) + n_big;
  else
    h.s_w = (const uint8_t*)a.s_w + (n_big / 128) * (a.K / KBYTES) * (a.s_w_fmt == 0 ? 4 : 1);
  h.y = (uint8_t*)a.y + n_big * (a.y_dtype == 0 ? 2 : 4);
  launch_cfg_sch<Half>(h, sch, code, stream);
  return hipGetLastError();
}

}  // namespace fgb
