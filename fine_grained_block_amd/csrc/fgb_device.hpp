// fgb_device.hpp — device-side fp8 codec and helpers for gfx950 (CDNA4).
//
// Formats (vLLM "FP8 W8A8", "Two FP8 representations"; IEEE-style per SqueezeBits "FP8
// Quantization with OwLite", "What is FP8 format"):
//   E4M3  s|eeee|mmm, bias 7, max +-448, NaN = S.1111.111, no inf, subnormal step 2^-9.
//   E5M2  s|eeeee|mm, bias 15, max +-57344, +-inf, NaN, subnormal step 2^-16.
//   UE8M0 (Transformers "Fine-grained FP8", "UE8M0 scale format"): 2^(c-127), 0xFF NaN.
// gfx950 implements the OCP E4M3/E5M2 encodings in hardware (v_cvt_pk_fp8_f32 and friends);
// these match the formats above.  The hardware converts with round-to-nearest-even; values are
// clamped to +-448 first, which is the saturation rule.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgb {

constexpr int kBlock = 128;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float32 -> bf16 bits, round-to-nearest-even (finite inputs; NaN kept quiet).
__host__ __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------------------------
// Integer reference encoders (exact by construction; used by the codec kernels and to check the
// hardware conversion).
// ---------------------------------------------------------------------------------------------
// E4M3, RNE, saturating to +-448.  Finite input.
__device__ __forceinline__ uint32_t enc_e4m3_sat_int(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {              // |x| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {        // |x| < 2^-6: subnormal E4M3 step 2^-9
    float t = __uint_as_float(a) * 512.0f;  // exact scaling
    code = (uint32_t)__builtin_rintf(t);    // 0..8 (8 is the smallest normal)
  } else {                              // normal: round the 23-bit mantissa to 3 bits, RNE
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);     // rebias 127 -> 7; a carry moves to the next binade
  }
  return code | sign;
}

// E5M2, RNE; saturate: clamp to +-57344 (inf too), else |x| >= 61440 -> inf; NaN -> 0x7F|s.
__device__ __forceinline__ uint32_t enc_e5m2_int(float x, bool saturate) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;
  } else if (a >= 0x47600000u) {       // |x| >= 57344 (inf included)
    code = saturate ? 0x7Bu : (a >= 0x47700000u ? 0x7Cu : 0x7Bu);  // 61440 = 0x47700000
  } else if (a < 0x38800000u) {        // |x| < 2^-14: subnormal step 2^-16
    float t = __uint_as_float(a) * 65536.0f;
    code = (uint32_t)__builtin_rintf(t);
  } else {
    uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
    code = (r >> 21) - (112u << 2);    // rebias 127 -> 15
  }
  return code | sign;
}

// Smallest power of two >= amax/448 as a UE8M0 code (clamped to 0..254); amax == 0 -> 127.
// amax = f * 2^p with f in [1, 2): amax/448 = (f/1.75) * 2^(p-8), so the exponent is p - 8 when
// f <= 1.75 (mantissa field <= 0x600000) and p - 7 otherwise.
__device__ __forceinline__ uint32_t ue8m0_from_amax(float amax) {
  uint32_t a = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (a == 0) return 127u;
  int e = (int)(a >> 23);  // biased exponent; 0 for subnormals (always clamps to code 0)
  if (e == 0) return 0u;
  int code = e - 8 + ((a & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return (uint32_t)(code < 0 ? 0 : (code > 254 ? 254 : code));
}

__device__ __forceinline__ float dec_ue8m0(uint32_t c) {
  c &= 0xFFu;
  if (c == 0xFFu) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(c == 0 ? 0x00400000u : (c << 23));  // c == 0: 2^-127 (subnormal)
}

__device__ __forceinline__ float dec_e4m3_int(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 15 && m == 7) return __uint_as_float(s | 0x7FC00000u);
  if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));  // m * 2^-9
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float dec_e5m2_int(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24, e = (c >> 2) & 0x1Fu, m = c & 3u;
  if (e == 31) return __uint_as_float(s | (m ? 0x7FC00000u : 0x7F800000u));
  if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 1.52587890625e-05f));  // m * 2^-16
  return __uint_as_float(s | ((e + 112u) << 23) | (m << 21));
}

// ---------------------------------------------------------------------------------------------
// Hardware E4M3 conversion of two values into bytes [2*hi .. 2*hi+1] of `old`, after clamping to
// +-448 (saturation).  v_cvt_pk_fp8_f32 rounds to nearest-even.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float clamp448(float r) {
  return __builtin_amdgcn_fmed3f(r, -kE4M3Max, kE4M3Max);
}

template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), (int)old, HI);
}

}  // namespace fgb
