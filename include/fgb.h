/*
 * fgb.h — fine-grained FP8 W8A8 block quantization and GEMM for AMD Instinct MI355X (gfx950).
 *
 * The scheme (Hugging Face Transformers, "Fine-grained FP8", intro and "DeepGEMM fast path"):
 * weights are E4M3 with one scale per 128x128 block; activations are quantized at run time
 * ("dynamic") per token in groups of 128 along the input dimension K; every FP8 linear is one
 * block-scaled GEMM, and MoE expert matmuls use a grouped variant.  Weight scales are float32
 * or packed UE8M0 powers of two ("UE8M0 scale format").  E4M3/E5M2 are defined on the vLLM
 * "FP8 W8A8" page, "Two FP8 representations".
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns every buffer.
 *     The library keeps no pointer after a call returns, allocates no device memory, and never
 *     synchronizes: work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   - Outputs must not alias inputs.
 *   - Validation is synchronous: an invalid argument returns a negative status before anything
 *     is enqueued.  There is no fallback path: a call either runs the gfx950 kernels or fails.
 *     (An explicitly requested backend that the hardware cannot run is an error, not a silent
 *     fallback: vLLM "FP8 W8A8", "GEMM kernel selection"; an unsupported scale format raises:
 *     Transformers "Fine-grained FP8", "UE8M0 scale format".)
 *   - Sizes and leading dimensions are in ELEMENTS.  Matrix and scale base pointers must be
 *     16-byte aligned and every row pitch in bytes a multiple of 16 (int32 expert offsets and
 *     status words: 4-byte aligned), else FGB_ERR_ALIGN.
 *   - M == 0 (or total_M == 0) is a valid no-op returning FGB_OK.
 *   - N and K must be multiples of 128 (the block edge), else FGB_ERR_SHAPE.
 *   - Inputs must be finite and codes must not be NaN (0x7F/0xFF); otherwise results are
 *     unspecified (no fault, but no meaning either).
 */
#ifndef FGB_H
#define FGB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FGB_ABI_VERSION 1
#define FGB_BLOCK 128

typedef enum {
  FGB_OK = 0,
  FGB_ERR_NULL = -1,      /* a required pointer is NULL */
  FGB_ERR_SHAPE = -2,     /* negative size, N or K not a multiple of 128, E <= 0, size too large */
  FGB_ERR_STRIDE = -3,    /* a leading dimension smaller than its row length */
  FGB_ERR_ALIGN = -4,     /* base pointer or row pitch not 16-byte aligned */
  FGB_ERR_ENUM = -5,      /* unknown enum value */
  FGB_ERR_WORKSPACE = -6, /* workspace NULL or smaller than the queried size */
  FGB_ERR_DEVICE = -7,    /* no current device, or the device is not gfx950 */
  FGB_ERR_LAUNCH = -8     /* the HIP runtime reported an error at launch */
} fgb_status;

typedef enum { FGB_SCALE_F32 = 0, FGB_SCALE_UE8M0 = 1 } fgb_scale_fmt; /* scale_fmt "float" | "ue8m0" */
typedef enum { FGB_OUT_BF16 = 0, FGB_OUT_F32 = 1 } fgb_out_dtype;      /* F32: diagnostic/test mode */
typedef enum {
  FGB_FP8_E4M3 = 0,     /* hardware conversion path used by the quantizers */
  FGB_FP8_E5M2 = 1,
  FGB_UE8M0 = 2,
  FGB_FP8_E4M3_INT = 3  /* encode only: integer bit-field encoder, to check the hardware path */
} fgb_fp8_fmt;

/* Activation and weight scale granularities of fgb_w8a8_scaled_gemm. */
typedef enum {
  FGB_ACT_SCALE_GROUP128 = 0, /* one scale per token per 1x128 group: fgb_w8a8_block_gemm */
  FGB_ACT_SCALE_TOKEN = 1,    /* one scale per token (row), float32 [M] */
  FGB_ACT_SCALE_TENSOR = 2    /* one scale for the whole tensor, float32 [1] */
} fgb_act_scale;
typedef enum {
  FGB_W_SCALE_BLOCK128 = 0, /* one scale per 128x128 block, [N/128, K/128] float32 or UE8M0 */
  FGB_W_SCALE_CHANNEL = 1   /* one scale per output feature (row of W), float32 [N] */
} fgb_w_scale;

/* Human-readable name of a status code (static storage; never NULL). */
const char* fgb_status_string(int status);

/* FGB_ABI_VERSION of the loaded library. */
int fgb_abi_version(void);

/*
 * Dynamic per-token, per-group activation quantization
 * (Transformers "Fine-grained FP8", intro: one scale per token per 128-group of K).
 *   x     bf16 bit patterns [M, ldx] row-major; group g of row m is x[m, 128g .. 128g+127].
 *   q     E4M3 codes [M, ldq] row-major (written for k < K).
 *   s_a   float32 scales, K-BLOCK-MAJOR: s_a[g * ld_sa + m], g < K/128, ld_sa >= M.
 * For every group: a = max|x| (exact); s = fl32(a / 448) (IEEE float32 division);
 * q = E4M3(fl32(x / s)) rounded to nearest-even and saturated to +-448; a == 0 gives s = 0 and
 * codes +-0 by the sign of x.  Results are bit-exact.
 * Requires K % 128 == 0, ldx >= K, ldq >= K, ld_sa >= M, ld_sa % 4 == 0.
 */
int fgb_act_quant_group128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                           uint8_t* q, int64_t ldq, float* s_a, int64_t ld_sa, void* stream);

/*
 * Per 128x128 block weight quantization (Transformers "Fine-grained FP8", intro;
 * "UE8M0 scale format" for fmt == FGB_SCALE_UE8M0).
 *   w     bf16 bit patterns [N, K] row-major (dense, ld = K).
 *   w_q   E4M3 codes [N, K] row-major.
 *   s_w   [N/128, K/128] row-major: float32 (FGB_SCALE_F32: s = fl32(amax/448)) or one byte per
 *         block (FGB_SCALE_UE8M0: the smallest power of two >= amax/448, code = log2(s) + 127,
 *         clamped to 0..254; amax == 0 gives code 127).  Codes are E4M3(fl32(w / s)), RNE,
 *         saturating.  Bit-exact.
 */
int fgb_weight_quant_block128(const uint16_t* w, int64_t N, int64_t K, uint8_t* w_q, void* s_w,
                              int s_w_fmt, void* stream);

/* Host query: workspace bytes fgb_w8a8_block_gemm needs for this shape (0 if none): the K-sliced
 * decode plans (16 < M <= 128) and the K-sliced prefill plan (prefill shapes with too few output tiles to
 * occupy the GPU, at most 32 MiB).  fgb_w8a8_scaled_gemm follows the same decode plan and needs
 * the workspace only for M <= 64. */
size_t fgb_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Block-scaled W8A8 GEMM (Transformers "Fine-grained FP8", "DeepGEMM fast path"; vLLM
 * "FP8 W8A8", intro: both operands 8-bit):
 *   y[m, n] = sum_kb s_a[kb*ld_sa + m] * s_w[n/128, kb] * sum_{k in kb} A_q[m, k] * W_q[n, k]
 * with every per-block product sum accumulated in float32 on the matrix cores, the scaled sum
 * over K-blocks in float32, and the result rounded to bf16 (RNE) or stored as float32.
 *   a_q   E4M3 [M, lda] row-major;  s_a  float32 K-block-major [K/128, ld_sa], ld_sa >= M;
 *   w_q   E4M3 [N, K] row-major (the Linear layout; y = A . W^T), dense;
 *   s_w   [N/128, K/128] row-major, float32 or UE8M0 bytes per s_w_fmt;
 *   y     [M, ldy] row-major, bf16 bit patterns or float32 per y_dtype.
 * Size limits (FGB_ERR_SHAPE otherwise): K <= 32768; M*lda, N*K and (K/128)*ld_sa*4 below 2^32.
 * M <= 64, and 64 < M <= 128 with K <= 8192, select the decode (weight-streaming) kernels; for
 * 16 < M they may slice K.  Other shapes select the prefill (matrix-core tile) kernels; when their
 * output tiles would occupy fewer than half of the compute units (e.g. N = 4096 at M = 256), K is
 * sliced as well.  A
 * sliced shape needs `workspace` of fgb_gemm_workspace_bytes(M, N, K) bytes: device, 16-byte
 * aligned, float32 partial sums added in slice order by a second launch; contents on entry are
 * ignored; 0 bytes (NULL allowed) when the shape is not sliced; FGB_ERR_WORKSPACE if missing or
 * too small.
 */
int fgb_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                        const uint8_t* w_q, const void* s_w, int s_w_fmt,
                        void* y, int y_dtype, int64_t ldy,
                        int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fgb_w8a8_block_gemm without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as fgb_w8a8_block_gemm; the calls that need a workspace
 * (K-sliced decode and prefill plans) use a scratch array that the library owns instead: 32 MiB
 * per GPU, held until the process ends (every workspace fits: the decode plans need at most
 * 24.5 MiB, the prefill plan is capped at 32 MiB; a shape needing more returns
 * FGB_ERR_WORKSPACE).  Allocates nothing.  All calls on one GPU share that GPU's scratch, so
 * calls that may overlap on one GPU (different streams without ordering) race and must not be
 * issued; calls ordered on one stream are fine.  The scratch needs no initial contents.
 */
int fgb_w8a8_block_gemm_noalloc(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt,
                                void* y, int y_dtype, int64_t ldy,
                                int64_t M, int64_t N, int64_t K, void* stream);

/* Host query: workspace bytes fgb_w8a8_block_gemm_fused_quant needs (0 if none, and for shapes it
 * rejects). */
size_t fgb_gemm_fused_quant_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Dynamic activation quantization and the decode GEMM in one call (Transformers "Fine-grained
 * FP8", intro and "DeepGEMM fast path": activations quantized at run time per token in 1x128
 * groups): the result of fgb_act_quant_group128 followed by fgb_w8a8_block_gemm, for M <= 64
 * (FGB_ERR_SHAPE above), equal to it bit for bit in float32 and bf16.  For a few tokens (M <= 4
 * with K >= 4096, or M <= 8 with N*K <= 16 MiB) it is one launch of a GEMM that quantizes each 1x128 group of x
 * right before its MFMA with the same arithmetic (s = fl32(amax/448), codes E4M3(fl32(x/s))),
 * and the codes and scales are not written out; for more tokens the call quantizes into the
 * workspace and runs the decode GEMM on it (repeating the quantization in every workgroup would
 * cost more than the launch it saves).
 *   x    bf16 [M, ldx] row-major, ldx >= K (16-byte rows);
 *   w_q, s_w, s_w_fmt, y, y_dtype, ldy as for fgb_w8a8_block_gemm;
 *   workspace  device, 16-byte aligned, >= fgb_gemm_fused_quant_workspace_bytes(M, N, K) bytes
 *              (may be NULL when that is 0; FGB_ERR_WORKSPACE if missing or too small).
 */
int fgb_w8a8_block_gemm_fused_quant(const uint16_t* x, int64_t ldx, const uint8_t* w_q,
                                    const void* s_w, int s_w_fmt, void* y, int y_dtype, int64_t ldy,
                                    int64_t M, int64_t N, int64_t K, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Host query: workspace bytes fgb_grouped_w8a8_block_gemm needs (0 if none). */
size_t fgb_grouped_gemm_workspace_bytes(int64_t total_M, int64_t N, int64_t K, int32_t E);

/*
 * Grouped (MoE expert) block-scaled GEMM (Transformers "Fine-grained FP8", "DeepGEMM fast path"
 * and "UE8M0 scale format": expert matmuls over FP8 block weights).  Rows are sorted by
 * expert; expert e owns rows expert_offsets[e] .. expert_offsets[e+1]-1 and computes the
 * fgb_w8a8_block_gemm result with w_q + e*N*K and its own scales.
 *   a_q [total_M, lda]; s_a [K/128, ld_sa], ld_sa >= total_M;
 *   w_q [E, N, K]; s_w [E, N/128, K/128] (float32 or UE8M0 bytes);
 *   expert_offsets  DEVICE int32 [E+1], offsets[0] == 0, nondecreasing, offsets[E] == total_M
 *                   (a precondition: checking it would need a device synchronization);
 *   total_M         host copy of offsets[E];
 *   y [total_M, ldy].
 * Experts with no rows are legal and write nothing.  1 <= E <= 65535.  Size limits as for
 * fgb_w8a8_block_gemm (per expert for W).
 */
int fgb_grouped_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt,
                                const int32_t* expert_offsets, int32_t E, int64_t total_M,
                                void* y, int y_dtype, int64_t ldy, int64_t N, int64_t K,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Masked batched MoE layout (Transformers "Fine-grained FP8", "UE8M0 scale format": the
 * batched_mm experts backend): every expert e has a slot of max_M rows, rows e*max_M ..
 * e*max_M + counts[e] - 1 of a_q / s_a / y, and only its first counts[e] rows are computed and
 * written (the rest of the slot is padding: never read into a stored result, never written).
 *   a_q [E*max_M, lda]; s_a [K/128, ld_sa], ld_sa >= E*max_M (one fgb_act_quant_group128 over all
 *   E*max_M rows gives both); w_q [E, N, K]; s_w [E, N/128, K/128] float32 or UE8M0;
 *   counts DEVICE int32 [E], 0 <= counts[e] <= max_M (a precondition; values are clamped to it);
 *   y [E*max_M, ldy].
 * max_M <= 64 runs the weight-streaming decode kernel per expert (the workgroups of an expert
 * with no rows exit at once, so only routed experts' weights are read); larger slots run the
 * grouped prefill kernel.  No workspace.  Size limits as for fgb_grouped_w8a8_block_gemm.
 * (fgb_grouped_w8a8_block_gemm also takes the weight-streaming path when total_M <= 64.)
 */
int fgb_batched_w8a8_block_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int64_t ld_sa,
                                const uint8_t* w_q, const void* s_w, int s_w_fmt,
                                const int32_t* counts, int32_t E, int64_t max_M,
                                void* y, int y_dtype, int64_t ldy, int64_t N, int64_t K, void* stream);

/*
 * Debugging aid for the grouped GEMM's precondition (the expert layout of Transformers
 * "Fine-grained FP8": rows sorted by expert, expert e owning rows offsets[e] .. offsets[e+1]-1).
 * Writes to `result` (DEVICE int32, 4-byte aligned; read it after synchronizing the stream) 0
 * when expert_offsets[0] == 0, the offsets are nondecreasing and expert_offsets[E] == total_M,
 * otherwise 1 + the first index i in 0..E whose entry breaks that.  Reads the E+1 offsets only.
 * FGB_ERR_SHAPE for E outside 1..65535 or total_M < 0, FGB_ERR_NULL, FGB_ERR_ALIGN as usual.
 */
int fgb_check_expert_offsets(const int32_t* expert_offsets, int32_t E, int64_t total_M, int32_t* result,
                             void* stream);

/*
 * The other FP8 schemes.  FP8_DYNAMIC (vLLM "FP8 W8A8", "Quantization process": static
 * per-channel weights, dynamic per-token activations, round-to-nearest); static activation
 * quantization with a given per-tensor scale (Transformers "Fine-grained FP8", "DeepGEMM fast
 * path"); E5M2 codes (vLLM "FP8 W8A8", "Two FP8 representations").  code_fmt is FGB_FP8_E4M3 or
 * FGB_FP8_E5M2; every scale divides by that format's maximum (448 or 57344); codes are
 * E(fl32(x / s)) rounded to nearest-even and saturated to the format's maximum; a scale of 0 (an
 * all-zero row or block) gives codes +-0 by sign.  Bit-exact.  Other rules as above
 * (FGB_ERR_ENUM for an unknown or unsupported format).
 */

/* Per-token activation quantization: s_a[m] = fl32(max_k |x[m, k]| / max) over the whole row.
 *   x bf16 [M, ldx]; q [M, ldq]; s_a float32 [M] (4-byte aligned).  K % 128 == 0. */
int fgb_act_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int code_fmt,
                            uint8_t* q, int64_t ldq, float* s_a, void* stream);

/* Per-output-channel weight quantization: s_w[n] = fl32(max_k |w[n, k]| / max) over row n of
 * the dense bf16 [N, K] weight; w_q [N, K]; s_w float32 [N].  N and K multiples of 128. */
int fgb_weight_quant_per_channel(const uint16_t* w, int64_t N, int64_t K, int code_fmt,
                                 uint8_t* w_q, float* s_w, void* stream);

/* Quantization with a given per-tensor scale: q = E(fl32(x / scale[0])).
 *   scale: DEVICE float32 [1], finite and > 0 (its value is a precondition: read on the
 *   device, not checked); x bf16 [M, ldx]; q [M, ldq].  K % 128 == 0. */
int fgb_act_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* scale,
                         int code_fmt, uint8_t* q, int64_t ldq, void* stream);

/* fgb_weight_quant_block128 with a choice of code format: E5M2 codes take float32 scales
 * amax/57344 (s_w_fmt FGB_SCALE_F32 only); E4M3 codes as fgb_weight_quant_block128. */
int fgb_weight_quant_block128_ex(const uint16_t* w, int64_t N, int64_t K, int code_fmt,
                                 uint8_t* w_q, void* s_w, int s_w_fmt, void* stream);

/*
 * GEMM under those scales, both operands in code_fmt (E4M3 x E4M3 or E5M2 x E5M2):
 *   act_scale TOKEN:  a(m) = s_a[m] (float32 [M]);  TENSOR: a(m) = s_a[0] (float32 [1]);
 *   w_scale CHANNEL:  y[m, n] = a(m) * s_w[n] * sum_k A_q[m, k] * W_q[n, k]   (s_w float32 [N],
 *                     16-byte aligned);
 *   w_scale BLOCK128: y[m, n] = a(m) * sum_kb s_w[n/128, kb] * sum_{k in kb} A_q[m, k] W_q[n, k]
 *                     (s_w [N/128, K/128] float32, or UE8M0 with E4M3 codes).
 * Products are summed in float32 on the matrix cores; scales that do not vary along K multiply
 * the float32 sum once at the end.  a_q [M, lda]; w_q [N, K] dense; y [M, ldy] bf16 or float32.
 * act_scale GROUP128 is FGB_ERR_ENUM here (that is fgb_w8a8_block_gemm).  Size limits, the
 * decode kernels (M <= 64) and the workspace as for fgb_w8a8_block_gemm: workspace device,
 * 16-byte aligned, >= fgb_gemm_workspace_bytes(M, N, K) bytes (NULL when that is 0;
 * FGB_ERR_WORKSPACE if missing or too small); the sliced decode calls add their float32 partials
 * in a second launch that also applies the scales.
 */
int fgb_w8a8_scaled_gemm(const uint8_t* a_q, int64_t lda, const float* s_a, int act_scale,
                         const uint8_t* w_q, const void* s_w, int w_scale, int s_w_fmt, int code_fmt,
                         void* y, int y_dtype, int64_t ldy, int64_t M, int64_t N, int64_t K,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Element-wise codecs (vLLM "FP8 W8A8", "Two FP8 representations"; UE8M0 per Transformers
 * "Fine-grained FP8", "UE8M0 scale format").
 *   encode: float32 in[n] -> u8 out[n].  E4M3: RNE, saturating to +-448 (`saturate` ignored).
 *           E5M2: RNE; saturate != 0 clamps to +-57344, else overflow gives +-inf.
 *           UE8M0: the smallest power of two >= in/448 (the weight-scale rule), in >= 0.
 *   decode: u8 in[n] -> float32 out[n] (E4M3, E5M2, UE8M0 = 2^(c-127), 0xFF = NaN).
 */
int fgb_fp8_encode(const float* in, uint8_t* out, int64_t n, int fmt, int saturate, void* stream);
int fgb_fp8_decode(const uint8_t* in, float* out, int64_t n, int fmt, void* stream);

/*
 * Self-test of the quantizers' division.  The codes are defined with the IEEE float32 quotient
 * x / s; the kernels form it as a correctly rounded reciprocal of s plus one FMA correction per
 * element, which is the IEEE quotient except where the FMA residual leaves the float32 normal
 * range (tiny x only; the quotient is then below 2^-13 and encodes as +-0 either way).  This
 * call checks, for every positive finite bf16 amax and every bf16 x with |x| <= amax (both
 * signs; about 1.07e9 pairs), s = fl32(amax/448) and both quotients, and ADDS to the device
 * counters: counts[0] += pairs whose E4M3 codes differ, counts[1] += pairs whose float32
 * quotients differ in any bit, counts[2] += those of them whose IEEE quotient has magnitude
 * >= 2^-13.  counts: device, 3 x uint64, 8-byte aligned; the caller zeroes them.
 */
int fgb_selftest_quotients(unsigned long long* counts, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FGB_H */
