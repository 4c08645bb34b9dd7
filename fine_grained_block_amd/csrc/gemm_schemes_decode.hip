// gemm_schemes_decode.hip — launches of the decode (M <= 64) kernels for the scaling schemes
// other than 1x128 groups x 128x128 blocks (see gemm_schemes_prefill.hip), with the block path's
// kernel selection and workspace plan: M <= 16 the register kernel, or the per-wave LDS-ring
// kernel for large weights with long rows; 16 < M <= 64 the per-wave ring kernel with 32 or 64
// activation rows for weights of at most 16 MiB, else the shared-ring kernel over K slices whose
// float32 partials the ordered reduction adds and scales.  Measured (graph loop, FP8_DYNAMIC E4M3,
// per-channel weights) against the per-wave ring kernel at every size, which these calls took
// before: 24576x1536 at M = 1 15.6 -> 8.2 us, 28672x4096 at M = 1 30.6 -> 22.8 us and at M = 64
// 53.5 -> 29.1 us, 7168x18432 at M = 64 55.0 -> 30.5 us; now within a few percent of the block
// scheme's decode at every decode shape and M.
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

template <int WK, int SCH, int SWF, int CODE>
void launch_small_sch(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N / 16)), block(64 * WK);
  if (a.y_dtype == 0)
    hipLaunchKernelGGL((gemm_decode_small_kernel<WK, SWF, 0, 0, SCH, CODE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_decode_small_kernel<WK, SWF, 1, 0, SCH, CODE>), grid, block, 0, stream, a);
}

template <int NW, int MT, int D, int SCH, int SWF, int CODE>
void launch_mid_nw(const GemmArgs& a, int kpw, int S, float* ws, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N / (16 * NW)) * S)), block(64 * NW);
  if (a.y_dtype == 0)
    hipLaunchKernelGGL((gemm_decode_mid_kernel<NW, MT, D, SWF, 0, SCH, CODE>), grid, block, 0, stream, a, kpw, S, ws);
  else
    hipLaunchKernelGGL((gemm_decode_mid_kernel<NW, MT, D, SWF, 1, SCH, CODE>), grid, block, 0, stream, a, kpw, S, ws);
}

template <int MT, int SCH, int SWF, int CODE>
void launch_mid_sch(const GemmArgs& a, void* workspace, hipStream_t stream) {
  const int S = decode_splits(a.M, a.N, a.K);
  const int nw = mid_waves(a.M, a.N, a.K);
  const int kpw = S == 1 ? (int)(a.K / 128) : mid_kpw(a.N, a.K);
  float* ws = reinterpret_cast<float*>(workspace);
  // (mid_waves returns 2 or 4 only for at most 32 activation rows)
  if (MT == 2 && nw == 2) launch_mid_nw<2, 2, 6, SCH, SWF, CODE>(a, kpw, S, ws, stream);
  else if (MT == 2 && nw == 4) launch_mid_nw<4, 2, 4, SCH, SWF, CODE>(a, kpw, S, ws, stream);
  else launch_mid_nw<8, MT, kMidStages, SCH, SWF, CODE>(a, kpw, S, ws, stream);
  if (S == 1) return;
  const int64_t total = a.M * (a.N / 4);
  const dim3 rgrid((unsigned)((total + 255) / 256));
  const float* s_w = reinterpret_cast<const float*>(a.s_w);
  if (a.y_dtype == 0)
    hipLaunchKernelGGL((splitk_reduce_kernel<0, SCH>), rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy, a.s_a,
                       a.a_kind, s_w);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<1, SCH>), rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy, a.s_a,
                       a.a_kind, s_w);
}

template <int SCH, int SWF, int CODE>
void launch_rows(const GemmArgs& a, void* workspace, hipStream_t stream) {
  if (a.M <= 16) {
    const int wk = decode_small_waves(a.N, a.K);
    if (decode_ring(a.N, a.K)) {
#define FGB_RING_SCH(WK)                                                   \
  do {                                                                     \
    if (a.M <= 8) launch_ring_sch<WK, 8, 5, SCH, SWF, CODE>(a, stream);    \
    else launch_ring_sch<WK, 16, 4, SCH, SWF, CODE>(a, stream);            \
  } while (0)
      if (wk == 8) FGB_RING_SCH(8);
      else if (wk == 4) FGB_RING_SCH(4);
      else if (wk == 2) FGB_RING_SCH(2);
      else FGB_RING_SCH(1);
#undef FGB_RING_SCH
    } else {
      if (wk == 8) launch_small_sch<8, SCH, SWF, CODE>(a, stream);
      else if (wk == 4) launch_small_sch<4, SCH, SWF, CODE>(a, stream);
      else if (wk == 2) launch_small_sch<2, SCH, SWF, CODE>(a, stream);
      else launch_small_sch<1, SCH, SWF, CODE>(a, stream);
    }
  } else if (!ring_mid_rows(a.N, a.K)) {
    if (a.M <= 32) launch_mid_sch<2, SCH, SWF, CODE>(a, workspace, stream);
    else launch_mid_sch<4, SCH, SWF, CODE>(a, workspace, stream);
  } else if (a.M <= 32) {
    launch_ring_sch<4, 32, 3, SCH, SWF, CODE>(a, stream);
  } else {
    launch_ring_sch<4, 64, 2, SCH, SWF, CODE>(a, stream);
  }
}

}  // namespace

hipError_t launch_gemm_scaled_decode(const GemmArgs& a, int sch, int code, void* workspace, hipStream_t stream) {
  if (sch == 2) {
    if (code == 0) launch_rows<2, 0, 0>(a, workspace, stream);
    else launch_rows<2, 0, 1>(a, workspace, stream);
  } else if (a.s_w_fmt == 0) {
    if (code == 0) launch_rows<1, 0, 0>(a, workspace, stream);
    else launch_rows<1, 0, 1>(a, workspace, stream);
  } else {
    launch_rows<1, 1, 0>(a, workspace, stream);
  }
  return hipGetLastError();
}

}  // namespace fgb
