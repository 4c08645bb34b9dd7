// quant_common.hpp — the quantizers' per-group arithmetic, shared by the quantization kernels
// and the GEMM that quantizes its activations itself: the scale's divisor and the quotient
// x / s, and the E4M3 encoding of 8 bf16 values.  (Scheme: Transformers "Fine-grained FP8",
// intro and "DeepGEMM fast path"; s = fl32(amax / 448), codes E4M3(fl32(x / s)), RNE, saturating.)
#pragma once
#include "fgb_device.hpp"

namespace fgb {

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15), via four DPP moves:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Max over the 8 lanes of a DPP half-row (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror).
__device__ __forceinline__ float row8_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// Max of non-negative values over groups of L consecutive lanes (L = 8, 16, 32 or 64), returned
// to every lane of the group: DPP within 16-lane rows, then the rows' maxima read with
// v_readlane and compared as integers (non-negative floats order like their bit patterns).
template <int L>
__device__ __forceinline__ float group_max_nonneg(float v) {
  static_assert(L == 8 || L == 16 || L == 32 || L == 64, "8, 16, 32 or 64 lanes");
  if constexpr (L == 8) return row8_max(v);
  v = row16_max(v);
  if constexpr (L == 16) return v;
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(v), 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(v), 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(v), 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(v), 48);
  if constexpr (L == 32) {
    const uint32_t lo = r0 > r1 ? r0 : r1, hi = r2 > r3 ? r2 : r3;
    return __uint_as_float((threadIdx.x & 32) ? hi : lo);
  } else {
    const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
    return __uint_as_float(a > b ? a : b);
  }
}

// Group divisor: the stored scale s, or 1 for an all-zero group (every x is +-0 there and the
// code keeps the sign).  `r` is the correctly rounded reciprocal 1/d, `fast` says whether d is in
// the range where the reciprocal-and-correct quotient below equals the IEEE quotient x/d.
struct Divisor {
  float d, r;
  bool fast;
};

__device__ __forceinline__ Divisor make_divisor(float s) {
  Divisor v;
  v.d = (s == 0.0f) ? 1.0f : s;
  v.r = 1.0f / v.d;  // IEEE division, correctly rounded
  // 2^-100 <= d <= 2^100: reciprocal, products and residuals stay clear of under/overflow
  const uint32_t e = (__float_as_uint(v.d) >> 23) & 0xFFu;
  v.fast = e >= 27u && e <= 227u;
  return v;
}

// fl32(x / d) without a division per element (Markstein, 1990; Muller et al., Handbook of
// Floating-Point Arithmetic): with r = RN(1/d) and q0 = RN(x r), the residual x - q0 d is computed
// in one FMA, and RN(q0 + residual * r) is the correctly rounded quotient whenever that residual
// is exact.  It is not exact when it falls below the float32 normal range, which happens only for
// tiny x: over every bf16 (x, amax) pair with |x| <= amax about 2.0e6 of 1.07e9 quotients differ
// from x / d in the last bit, all of them with |x / d| < 2^-13, far below 2^-10, under which
// every value encodes as E4M3 +-0 — so the codes never differ.  Outside the fast range of d the
// IEEE division is used.  fgb_selftest_quotients checks all of this exhaustively on the device.
__device__ __forceinline__ float quot_fast(float x, const Divisor& v) {
  const float q0 = x * v.r;
  const float e = __builtin_fmaf(-q0, v.d, x);
  // d > 0, so the quotient has x's sign; the correction step would turn x = -0 into +0
  return __builtin_copysignf(__builtin_fmaf(e, v.r, q0), x);
}

__device__ __forceinline__ float quot(float x, const Divisor& v) { return v.fast ? quot_fast(x, v) : x / v.d; }

// Quantize 8 values (4 bf16 pairs) by divisor v.  Returns 8 E4M3 codes in two dwords.  All
// lanes of the wave must be active (the fast/slow choice is made for the whole wave).
__device__ __forceinline__ uint2 quant8(const uint4 w, const Divisor& v) {
  float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  if (__all(v.fast)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = quot_fast(f[i], v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = quot(f[i], v);
  }
  uint32_t lo = cvt_pk_e4m3<false>(f[0], f[1], 0u);
  lo = cvt_pk_e4m3<true>(f[2], f[3], lo);
  uint32_t hi = cvt_pk_e4m3<false>(f[4], f[5], 0u);
  hi = cvt_pk_e4m3<true>(f[6], f[7], hi);
  return make_uint2(lo, hi);
}

__device__ __forceinline__ float absmax8(const uint4 v) {
  float a = fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x)));
  float b = fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)));
  float c = fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z)));
  float d = fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

}  // namespace fgb
