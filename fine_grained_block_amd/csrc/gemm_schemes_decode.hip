// gemm_schemes_decode.hip — launches of the per-wave ring decode kernel (M <= 64) for the scaling
// schemes other than 1x128 groups x 128x128 blocks (see gemm_schemes_prefill.hip): one launch,
// no workspace; 8, 16, 32 or 64 staged activation rows.
#include "gemm_decode_kernels.hpp"

namespace fgb {

namespace {

template <int WK, int MR, int D, int SCH, int SWF, int CODE>
void launch_ring_sch(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N / 16)), block(64 * WK);
  if (a.y_dtype == 0)
    hipLaunchKernelGGL((gemm_decode_ring_kernel<WK, MR, D, SWF, 0, SCH, CODE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_decode_ring_kernel<WK, MR, D, SWF, 1, SCH, CODE>), grid, block, 0, stream, a);
}

template <int SCH, int SWF, int CODE>
void launch_rows(const GemmArgs& a, hipStream_t stream) {
  if (a.M <= 8) launch_ring_sch<8, 8, 5, SCH, SWF, CODE>(a, stream);
  else if (a.M <= 16) launch_ring_sch<8, 16, 4, SCH, SWF, CODE>(a, stream);
  else if (a.M <= 32) launch_ring_sch<4, 32, 3, SCH, SWF, CODE>(a, stream);
  else launch_ring_sch<4, 64, 2, SCH, SWF, CODE>(a, stream);
}

}  // namespace

hipError_t launch_gemm_scaled_decode(const GemmArgs& a, int sch, int code, hipStream_t stream) {
  if (sch == 2) {
    if (code == 0) launch_rows<2, 0, 0>(a, stream);
    else launch_rows<2, 0, 1>(a, stream);
  } else if (a.s_w_fmt == 0) {
    if (code == 0) launch_rows<1, 0, 0>(a, stream);
    else launch_rows<1, 0, 1>(a, stream);
  } else {
    launch_rows<1, 1, 0>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace fgb
