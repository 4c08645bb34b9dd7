// internal.h — launchers shared between the kernel sources and the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fgb {

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* s_a, int64_t ld_sa, hipStream_t stream);
hipError_t launch_weight_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq, void* s_w,
                               int fmt, hipStream_t stream, int code = 0);
// one scale per row over the whole row (per-token activations, per-channel weights)
hipError_t launch_row_quant(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* s, int code, hipStream_t stream);
// a given per-tensor scale (device float)
hipError_t launch_static_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* scale,
                               uint8_t* q, int64_t ldq, int code, hipStream_t stream);
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
  // other scaling schemes: the activation scale is per token (s_a[m], 1) or one for the tensor
  // (s_a[0], 2); 0 = per 1x128 group (s_a K-block-major)
  int a_kind;
  // masked batched MoE layout (grouped only): expert e owns rows e*slot .. e*slot + counts[e] - 1,
  // counts[e] read from `offsets` (then E entries); 0 = contiguous rows from offsets [E+1]
  int64_t slot;
  // K-sliced prefill launch only: K-blocks per slice (slice y starts at K-block y*kslice)
  int kslice;
};

// Prefill (M > 64) dense GEMM and the grouped variant.  Launches with too few output tiles to
// occupy the CUs (M a little above the decode sizes, narrow N) slice K: float32 partials in
// `workspace` (prefill_workspace_bytes), added in slice order by a second launch.
int prefill_splits(int64_t M, int64_t N, int64_t K);
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_prefill(const GemmArgs& a, void* workspace, hipStream_t stream);
// y[m, n] = sum over s of ws[s][m][n] in slice order, as bf16 (y_dtype 0) or float32
hipError_t launch_splitk_reduce(const float* ws, int S, int64_t M, int64_t N, void* y, int y_dtype, int64_t ldy,
                                hipStream_t stream);
// compute units of the current device; output columns of a dense prefill GEMM (N % 256 == 0) that
// run as 256 x 256 tiles (the rest as 256 x 128 tiles)
int cu_count();
int64_t big_columns(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t stream);
hipError_t launch_check_offsets(const int32_t* offsets, int32_t E, int64_t total_M, int32_t* result,
                                hipStream_t stream);

// The other scaling schemes (sch 1: per-token or per-tensor activation scale with 128x128 weight
// blocks; sch 2: per-channel weight scales), E4M3 (code 0) or E5M2 (code 1) operands.
hipError_t launch_gemm_scaled_prefill(const GemmArgs& a, int sch, int code, hipStream_t stream);
hipError_t launch_gemm_scaled_decode(const GemmArgs& a, int sch, int code, void* workspace, hipStream_t stream);

// MoE with at most 64 rows per expert: mode 1 grouped (offsets [E+1]), mode 2 batched (counts [E],
// slot rows per expert).
hipError_t launch_gemm_moe_decode(const GemmArgs& a, int mode, hipStream_t stream);

// act_quant + decode GEMM from bf16 activations (M <= 64): one launch of the GEMM that quantizes
// its activations itself where that is faster (workspace 0), else act_quant into the workspace
// and the decode GEMM.
size_t fused_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_decode_fused(const GemmArgs& a, const uint16_t* x, int64_t ldx, void* workspace,
                                    hipStream_t stream);
hipError_t launch_gemm_decode_fused_small(const GemmArgs& a, const uint16_t* x, int64_t ldx, hipStream_t stream);
// waves per 16-row workgroup that split K in the M <= 16 decode kernels
int decode_small_waves(int64_t N, int64_t K);

// Whether the block GEMM takes the decode (weight-streaming) kernels: up to 64 rows, and 65-128
// rows when K has at most 64 blocks (the shared-ring kernel with 128 activation rows); otherwise
// the prefill tiles.  Measured (graph loop) at 65 / 128 rows against the K-sliced prefill launch:
// 4096x4096 13.9 / 16.2 vs 16.7 / 21.4 us, 6144x4096 15.3 / 19.3 vs 17.3 / 21.3, 24576x1536
// 15.3 / 16.2 vs 17.0 / 18.3, 28672x4096 35.6 / 35.5 vs 34.4 / 40.2; with long rows the prefill
// slices were ahead (7168x18432 42.7 / 43.9 vs 34.7 / 39.7 us, 4096x14336 23.5 / 25.9 vs 22.6 / 27.3).
constexpr int64_t kDecodeMaxM = 128;
constexpr bool use_decode(int64_t M, int64_t K) { return M <= 64 || (M <= kDecodeMaxM && K <= 64 * 128); }

// Decode path selection (M <= kDecodeMaxM): the LDS-ring kernel for M <= 16 (large weights, long rows);
// the per-wave ring kernel for 16 < M <= 64 (small weights); the K-blocks per workgroup of the
// shared-ring 16 < M <= 128 kernel and its number of slices (> 1: partials and a second launch).
bool decode_ring(int64_t N, int64_t K);
bool ring_mid_rows(int64_t N, int64_t K);
int mid_kpw(int64_t N, int64_t K);
constexpr int kMidStages = 4;  // LDS stages of the shared-ring kernel (measured: 4 >= 5, 6)
int mid_waves(int64_t M, int64_t N, int64_t K);
int decode_splits(int64_t M, int64_t N, int64_t K);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_decode(const GemmArgs& a, void* workspace, hipStream_t stream);

// Scratch that the library owns for callers that cannot allocate: kScratchBytes per GPU.  It
// covers every workspace of the GEMM: the decode plans need at most 128 x 49024 float32 partials
// (24.5 MiB), and the K-sliced prefill plan is capped at this size.
constexpr size_t kScratchBytes = (size_t)32 << 20;
// The current device's scratch address (looked up once per device).
hipError_t scratch_address(void** out);

}  // namespace fgb
