// api.cpp — the C-ABI of libfgb: argument validation, device check, path selection, launches.
//
// Validation is synchronous and happens before anything is enqueued; there is no fallback
// path (an unsupported request is an error: vLLM "FP8 W8A8", "GEMM kernel selection"; an
// unsupported scale format raises: Transformers "Fine-grained FP8", "UE8M0 scale format").
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../include/fgb.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // grid and index arithmetic bound
constexpr int64_t kMax32 = (int64_t)1 << 32;   // bytes addressable by a 32-bit offset
constexpr int kMaxDevices = 64;
constexpr int kMaxExperts = 65535;  // experts index grid.y in the per-expert decode kernels

// 0 = unknown, 1 = gfx950, -1 = other
int g_dev_ok[kMaxDevices];

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FGB_ERR_DEVICE;
  }
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FGB_ERR_DEVICE;
    }
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return g_dev_ok[dev] == 1 ? FGB_OK : FGB_ERR_DEVICE;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FGB_OK : FGB_ERR_LAUNCH; }

// Shared validation of the GEMM operands (dense: E = 1, offsets unused).
int validate_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                  const uint8_t* w_q, const void* s_w, int s_w_fmt, const void* y, int y_dtype,
                  int64_t ldy, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FGB_ERR_SHAPE;
  if (N % FGB_BLOCK || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (s_w_fmt != FGB_SCALE_F32 && s_w_fmt != FGB_SCALE_UE8M0) return FGB_ERR_ENUM;
  if (y_dtype != FGB_OUT_BF16 && y_dtype != FGB_OUT_F32) return FGB_ERR_ENUM;
  if (M == 0) return FGB_OK;
  if (!a_q || !s_a || !w_q || !s_w || !y) return FGB_ERR_NULL;
  if (lda < K || ldy < N || ld_sa < M) return FGB_ERR_STRIDE;
  const int64_t ybytes = y_dtype == FGB_OUT_BF16 ? 2 : 4;
  if (!aligned16(a_q) || !aligned16(s_a) || !aligned16(w_q) || !aligned16(s_w) || !aligned16(y))
    return FGB_ERR_ALIGN;
  if (lda % 16 || (ldy * ybytes) % 16 || (ld_sa * 4) % 16) return FGB_ERR_ALIGN;
  // the kernels address A, one expert's W and the scales with 32-bit offsets, and hold a weight
  // row's K/128 block scales in registers (K <= 32768)
  if (M * lda >= kMax32 || N * K >= kMax32 || (K / FGB_BLOCK) * ld_sa * 4 >= kMax32) return FGB_ERR_SHAPE;
  if (K > 32768) return FGB_ERR_SHAPE;
  return FGB_OK;
}

}  // namespace

extern "C" {

const char* fgb_status_string(int status) {
  switch (status) {
    case FGB_OK: return "FGB_OK";
    case FGB_ERR_NULL: return "FGB_ERR_NULL: a required pointer is NULL";
    case FGB_ERR_SHAPE: return "FGB_ERR_SHAPE: invalid size (N and K must be positive multiples of 128)";
    case FGB_ERR_STRIDE: return "FGB_ERR_STRIDE: leading dimension smaller than the row length";
    case FGB_ERR_ALIGN: return "FGB_ERR_ALIGN: pointer or row pitch not 16-byte aligned";
    case FGB_ERR_ENUM: return "FGB_ERR_ENUM: unknown enum value";
    case FGB_ERR_WORKSPACE: return "FGB_ERR_WORKSPACE: workspace missing or too small";
    case FGB_ERR_DEVICE: return "FGB_ERR_DEVICE: no current device or the device is not gfx950";
    case FGB_ERR_LAUNCH: return "FGB_ERR_LAUNCH: kernel launch failed";
    default: return "unknown fgb status";
  }
}

int fgb_abi_version(void) { return FGB_ABI_VERSION; }

int fgb_act_quant_group128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                           int64_t ldq, float* s_a, int64_t ld_sa, void* stream) {
  if (M < 0 || K <= 0 || M >= kMaxDim || K >= kMaxDim || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (M == 0) return FGB_OK;
  if (!x || !q || !s_a) return FGB_ERR_NULL;
  if (ldx < K || ldq < K || ld_sa < M) return FGB_ERR_STRIDE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s_a)) return FGB_ERR_ALIGN;
  if ((ldx * 2) % 16 || ldq % 16 || (ld_sa * 4) % 16) return FGB_ERR_ALIGN;
  if ((M * (K / FGB_BLOCK)) >= kMaxDim) return FGB_ERR_SHAPE;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_act_quant(x, M, K, ldx, q, ldq, s_a, ld_sa, (hipStream_t)stream));
}

int fgb_weight_quant_block128(const uint16_t* w, int64_t N, int64_t K, uint8_t* w_q, void* s_w,
                              int s_w_fmt, void* stream) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim || N % FGB_BLOCK || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (s_w_fmt != FGB_SCALE_F32 && s_w_fmt != FGB_SCALE_UE8M0) return FGB_ERR_ENUM;
  if (N == 0 || K == 0) return FGB_OK;
  if (!w || !w_q || !s_w) return FGB_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_q)) return FGB_ERR_ALIGN;
  if (s_w_fmt == FGB_SCALE_F32 && ((uintptr_t)s_w & 3u)) return FGB_ERR_ALIGN;
  if ((N / FGB_BLOCK) * (K / FGB_BLOCK) >= kMaxDim) return FGB_ERR_SHAPE;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_weight_quant(w, N, K, w_q, s_w, s_w_fmt, (hipStream_t)stream));
}

size_t fgb_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
  if (N % FGB_BLOCK || K % FGB_BLOCK) return 0;
  return fgb::use_decode(M, K) ? fgb::decode_workspace_bytes(M, N, K) : fgb::prefill_workspace_bytes(M, N, K);
}

int fgb_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                        const uint8_t* w_q, const void* s_w, int s_w_fmt, void* y, int y_dtype,
                        int64_t ldy, int64_t M, int64_t N, int64_t K, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = validate_gemm(a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K);
  if (st != FGB_OK || M == 0) return st;
  const bool decode = fgb::use_decode(M, K);
  const size_t need = decode ? fgb::decode_workspace_bytes(M, N, K) : fgb::prefill_workspace_bytes(M, N, K);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FGB_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return FGB_ERR_ALIGN;
  st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K, nullptr, 1};
  if (decode) return launch_status(fgb::launch_gemm_decode(a, workspace, (hipStream_t)stream));
  return launch_status(fgb::launch_gemm_prefill(a, workspace, (hipStream_t)stream));
}

int fgb_w8a8_block_gemm_noalloc(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt, void* y, int y_dtype,
                                int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = validate_gemm(a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K);
  if (st != FGB_OK || M == 0) return st;
  const bool decode = fgb::use_decode(M, K);
  const size_t need = decode ? fgb::decode_workspace_bytes(M, N, K) : fgb::prefill_workspace_bytes(M, N, K);
  if (need > fgb::kScratchBytes) return FGB_ERR_WORKSPACE;
  st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K, nullptr, 1};
  void* ws = nullptr;
  if (need > 0 && fgb::scratch_address(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return FGB_ERR_DEVICE;
  }
  if (!decode) return launch_status(fgb::launch_gemm_prefill(a, ws, (hipStream_t)stream));
  return launch_status(fgb::launch_gemm_decode(a, ws, (hipStream_t)stream));
}

int fgb_weight_quant_block128_ex(const uint16_t* w, int64_t N, int64_t K, int code_fmt, uint8_t* w_q, void* s_w,
                                 int s_w_fmt, void* stream) {
  if (code_fmt != FGB_FP8_E4M3 && code_fmt != FGB_FP8_E5M2) return FGB_ERR_ENUM;
  if (s_w_fmt != FGB_SCALE_F32 && s_w_fmt != FGB_SCALE_UE8M0) return FGB_ERR_ENUM;
  if (code_fmt == FGB_FP8_E5M2 && s_w_fmt != FGB_SCALE_F32) return FGB_ERR_ENUM;
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim || N % FGB_BLOCK || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (N == 0 || K == 0) return FGB_OK;
  if (!w || !w_q || !s_w) return FGB_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_q)) return FGB_ERR_ALIGN;
  if (s_w_fmt == FGB_SCALE_F32 && ((uintptr_t)s_w & 3u)) return FGB_ERR_ALIGN;
  if ((N / FGB_BLOCK) * (K / FGB_BLOCK) >= kMaxDim) return FGB_ERR_SHAPE;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_weight_quant(w, N, K, w_q, s_w, s_w_fmt, (hipStream_t)stream,
                                                code_fmt == FGB_FP8_E5M2 ? 1 : 0));
}

namespace {

// Per-row quantization (per token or per output channel): rows x K bf16 -> codes, one scale per row.
int row_quant(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, int code_fmt, uint8_t* q, int64_t ldq,
              float* s, void* stream) {
  if (code_fmt != FGB_FP8_E4M3 && code_fmt != FGB_FP8_E5M2) return FGB_ERR_ENUM;
  if (rows < 0 || K <= 0 || rows >= kMaxDim || K >= kMaxDim || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (rows == 0) return FGB_OK;
  if (!x || !q || !s) return FGB_ERR_NULL;
  if (ldx < K || ldq < K) return FGB_ERR_STRIDE;
  if (!aligned16(x) || !aligned16(q) || ((uintptr_t)s & 3u)) return FGB_ERR_ALIGN;
  if ((ldx * 2) % 16 || ldq % 16) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_row_quant(x, rows, K, ldx, q, ldq, s, code_fmt == FGB_FP8_E5M2 ? 1 : 0,
                                             (hipStream_t)stream));
}

}  // namespace

int fgb_act_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int code_fmt, uint8_t* q,
                            int64_t ldq, float* s_a, void* stream) {
  return row_quant(x, M, K, ldx, code_fmt, q, ldq, s_a, stream);
}

int fgb_weight_quant_per_channel(const uint16_t* w, int64_t N, int64_t K, int code_fmt, uint8_t* w_q, float* s_w,
                                 void* stream) {
  if (N % FGB_BLOCK) return FGB_ERR_SHAPE;
  return row_quant(w, N, K, K, code_fmt, w_q, K, s_w, stream);
}

int fgb_act_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* scale, int code_fmt,
                         uint8_t* q, int64_t ldq, void* stream) {
  if (code_fmt != FGB_FP8_E4M3 && code_fmt != FGB_FP8_E5M2) return FGB_ERR_ENUM;
  if (M < 0 || K <= 0 || M >= kMaxDim || K >= kMaxDim || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (M == 0) return FGB_OK;
  if (!x || !q || !scale) return FGB_ERR_NULL;
  if (ldx < K || ldq < K) return FGB_ERR_STRIDE;
  if (!aligned16(x) || !aligned16(q) || ((uintptr_t)scale & 3u)) return FGB_ERR_ALIGN;
  if ((ldx * 2) % 16 || ldq % 16) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_static_quant(x, M, K, ldx, scale, q, ldq, code_fmt == FGB_FP8_E5M2 ? 1 : 0,
                                                (hipStream_t)stream));
}

int fgb_w8a8_scaled_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int act_scale, const uint8_t* w_q,
                         const void* s_w, int w_scale, int s_w_fmt, int code_fmt, void* y, int y_dtype, int64_t ldy,
                         int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FGB_ERR_SHAPE;
  if (N % FGB_BLOCK || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (act_scale != FGB_ACT_SCALE_TOKEN && act_scale != FGB_ACT_SCALE_TENSOR) return FGB_ERR_ENUM;
  if (w_scale != FGB_W_SCALE_BLOCK128 && w_scale != FGB_W_SCALE_CHANNEL) return FGB_ERR_ENUM;
  if (s_w_fmt != FGB_SCALE_F32 && s_w_fmt != FGB_SCALE_UE8M0) return FGB_ERR_ENUM;
  if (code_fmt != FGB_FP8_E4M3 && code_fmt != FGB_FP8_E5M2) return FGB_ERR_ENUM;
  if (s_w_fmt == FGB_SCALE_UE8M0 && (w_scale != FGB_W_SCALE_BLOCK128 || code_fmt != FGB_FP8_E4M3)) return FGB_ERR_ENUM;
  if (y_dtype != FGB_OUT_BF16 && y_dtype != FGB_OUT_F32) return FGB_ERR_ENUM;
  if (M == 0) return FGB_OK;
  if (!a_q || !s_a || !w_q || !s_w || !y) return FGB_ERR_NULL;
  if (lda < K || ldy < N) return FGB_ERR_STRIDE;
  const int64_t ybytes = y_dtype == FGB_OUT_BF16 ? 2 : 4;
  if (!aligned16(a_q) || !aligned16(w_q) || !aligned16(s_w) || !aligned16(y) || ((uintptr_t)s_a & 3u))
    return FGB_ERR_ALIGN;
  if (lda % 16 || (ldy * ybytes) % 16) return FGB_ERR_ALIGN;
  if (M * lda >= kMax32 || N * K >= kMax32 || K > 32768) return FGB_ERR_SHAPE;
  // the same decode plan (and workspace) as fgb_w8a8_block_gemm
  const size_t need = M <= 64 ? fgb::decode_workspace_bytes(M, N, K) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FGB_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{a_q, lda, s_a, 0, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K, nullptr, 1, act_scale};
  const int sch = w_scale == FGB_W_SCALE_CHANNEL ? 2 : 1;
  const int code = code_fmt == FGB_FP8_E5M2 ? 1 : 0;
  if (M <= 64) return launch_status(fgb::launch_gemm_scaled_decode(a, sch, code, workspace, (hipStream_t)stream));
  return launch_status(fgb::launch_gemm_scaled_prefill(a, sch, code, (hipStream_t)stream));
}

size_t fgb_gemm_fused_quant_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > 64 || N <= 0 || K <= 0 || N % FGB_BLOCK || K % FGB_BLOCK || K > 32768) return 0;
  return fgb::fused_workspace_bytes(M, N, K);
}

int fgb_w8a8_block_gemm_fused_quant(const uint16_t* x, int64_t ldx, const uint8_t* w_q, const void* s_w,
                                    int s_w_fmt, void* y, int y_dtype, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || M > 64 || N <= 0 || K <= 0 || N >= kMaxDim || K >= kMaxDim) return FGB_ERR_SHAPE;
  if (N % FGB_BLOCK || K % FGB_BLOCK) return FGB_ERR_SHAPE;
  if (s_w_fmt != FGB_SCALE_F32 && s_w_fmt != FGB_SCALE_UE8M0) return FGB_ERR_ENUM;
  if (y_dtype != FGB_OUT_BF16 && y_dtype != FGB_OUT_F32) return FGB_ERR_ENUM;
  if (M == 0) return FGB_OK;
  if (!x || !w_q || !s_w || !y) return FGB_ERR_NULL;
  if (ldx < K || ldy < N) return FGB_ERR_STRIDE;
  const int64_t ybytes = y_dtype == FGB_OUT_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(s_w) || !aligned16(y)) return FGB_ERR_ALIGN;
  if ((ldx * 2) % 16 || (ldy * ybytes) % 16) return FGB_ERR_ALIGN;
  if (M * ldx * 2 >= kMax32 || N * K >= kMax32 || K > 32768) return FGB_ERR_SHAPE;
  const size_t need = fgb::fused_workspace_bytes(M, N, K);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FGB_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{nullptr, 0, nullptr, 0, w_q, s_w, s_w_fmt, y, y_dtype, ldy, M, N, K, nullptr, 1, 0};
  return launch_status(fgb::launch_gemm_decode_fused(a, x, ldx, workspace, (hipStream_t)stream));
}

size_t fgb_grouped_gemm_workspace_bytes(int64_t total_M, int64_t N, int64_t K, int32_t E) {
  (void)total_M; (void)N; (void)K; (void)E;
  return 0;
}

int fgb_grouped_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt,
                                const int32_t* expert_offsets, int32_t E, int64_t total_M,
                                void* y, int y_dtype, int64_t ldy, int64_t N, int64_t K,
                                void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  if (E <= 0 || E > kMaxExperts) return FGB_ERR_SHAPE;
  int st = validate_gemm(a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, total_M, N, K);
  if (st != FGB_OK || total_M == 0) return st;
  if (!expert_offsets) return FGB_ERR_NULL;
  if (((uintptr_t)expert_offsets & 3u)) return FGB_ERR_ALIGN;
  // tile-count bound: (ceil(total_M/128) + E) * N/128 workgroups
  if (((total_M + 127) / 128 + E) * (N / 128) >= kMaxDim) return FGB_ERR_SHAPE;
  st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, total_M, N, K,
                  expert_offsets, E};
  // at most 64 rows in all (decode-shaped routing): the weight-streaming kernel per expert
  if (total_M <= 64) return launch_status(fgb::launch_gemm_moe_decode(a, 1, (hipStream_t)stream));
  return launch_status(fgb::launch_gemm_grouped(a, (hipStream_t)stream));
}

int fgb_batched_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt, const int32_t* counts,
                                int32_t E, int64_t max_M, void* y, int y_dtype, int64_t ldy, int64_t N, int64_t K,
                                void* stream) {
  if (E <= 0 || E > kMaxExperts || max_M < 0 || max_M >= kMaxDim) return FGB_ERR_SHAPE;
  const int64_t rows = (int64_t)E * max_M;
  if (rows >= kMaxDim) return FGB_ERR_SHAPE;
  int st = validate_gemm(a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, rows, N, K);
  if (st != FGB_OK || rows == 0) return st;
  if (!counts) return FGB_ERR_NULL;
  if (((uintptr_t)counts & 3u)) return FGB_ERR_ALIGN;
  // tile-count bound of the prefill form: E * ceil(max_M / 128) tile-rows
  if ((int64_t)E * ((max_M + 127) / 128) * (N / 128) >= kMaxDim) return FGB_ERR_SHAPE;
  st = check_device();
  if (st != FGB_OK) return st;
  fgb::GemmArgs a{a_q, lda, s_a, ld_sa, w_q, s_w, s_w_fmt, y, y_dtype, ldy, rows, N, K, counts, E, 0, max_M};
  if (max_M <= 64) return launch_status(fgb::launch_gemm_moe_decode(a, 2, (hipStream_t)stream));
  return launch_status(fgb::launch_gemm_grouped(a, (hipStream_t)stream));
}

int fgb_check_expert_offsets(const int32_t* expert_offsets, int32_t E, int64_t total_M, int32_t* result,
                             void* stream) {
  if (E <= 0 || E > kMaxExperts || total_M < 0) return FGB_ERR_SHAPE;
  if (!expert_offsets || !result) return FGB_ERR_NULL;
  if (((uintptr_t)expert_offsets & 3u) || ((uintptr_t)result & 3u)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_check_offsets(expert_offsets, E, total_M, result, (hipStream_t)stream));
}

int fgb_fp8_encode(const float* in, uint8_t* out, int64_t n, int fmt, int saturate, void* stream) {
  if (n < 0) return FGB_ERR_SHAPE;
  if (fmt < FGB_FP8_E4M3 || fmt > FGB_FP8_E4M3_INT) return FGB_ERR_ENUM;
  if (n == 0) return FGB_OK;
  if (!in || !out) return FGB_ERR_NULL;
  if (((uintptr_t)in & 3u)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_encode(in, out, n, fmt, saturate, (hipStream_t)stream));
}

int fgb_fp8_decode(const uint8_t* in, float* out, int64_t n, int fmt, void* stream) {
  if (n < 0) return FGB_ERR_SHAPE;
  if (fmt < FGB_FP8_E4M3 || fmt > FGB_UE8M0) return FGB_ERR_ENUM;
  if (n == 0) return FGB_OK;
  if (!in || !out) return FGB_ERR_NULL;
  if (((uintptr_t)out & 3u)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_decode(in, out, n, fmt, (hipStream_t)stream));
}

int fgb_selftest_quotients(unsigned long long* counts, void* stream) {
  if (!counts) return FGB_ERR_NULL;
  if (((uintptr_t)counts & 7u)) return FGB_ERR_ALIGN;
  int st = check_device();
  if (st != FGB_OK) return st;
  return launch_status(fgb::launch_selftest_quotients(counts, (hipStream_t)stream));
}

}  // extern "C"
