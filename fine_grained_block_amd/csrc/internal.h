// internal.h — launchers shared between the kernel sources and the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fgb {

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* s_a, int64_t ld_sa, hipStream_t stream);
hipError_t launch_weight_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq, void* s_w,
                               int fmt, hipStream_t stream);
hipError_t launch_encode(const float* in, uint8_t* out, int64_t n, int fmt, int saturate,
                         hipStream_t stream);
hipError_t launch_decode(const uint8_t* in, float* out, int64_t n, int fmt, hipStream_t stream);
hipError_t launch_selftest_quotients(unsigned long long* counts, hipStream_t stream);

// Block-scaled GEMM problem description (dense or grouped).
struct GemmArgs {
  const uint8_t* a_q;
  int64_t lda;
  const float* s_a;
  int64_t ld_sa;
  const uint8_t* w_q;
  const void* s_w;
  int s_w_fmt;  // 0 float32, 1 UE8M0
  void* y;
  int y_dtype;  // 0 bf16, 1 float32
  int64_t ldy;
  int64_t M, N, K;
  // grouped only
  const int32_t* offsets;
  int32_t E;
};

// Prefill (M > 64) dense GEMM and the grouped variant.
hipError_t launch_gemm_prefill(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t stream);
hipError_t launch_check_offsets(const int32_t* offsets, int32_t E, int64_t total_M, int32_t* result,
                                hipStream_t stream);

// Split-K decode path (M <= 64).
int decode_splits(int64_t M, int64_t N, int64_t K);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_decode(const GemmArgs& a, void* workspace, hipStream_t stream);

}  // namespace fgb
