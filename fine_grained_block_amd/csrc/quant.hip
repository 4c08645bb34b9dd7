// quant.hip — dynamic activation quantization (1x128 groups), 128x128 weight-block quantization
// and element-wise fp8 codec kernels for gfx950.
//
// Scheme: Transformers "Fine-grained FP8", intro (weights per 128x128 block, activations per
// token per group of 128 along K) and "DeepGEMM fast path" (activation scales computed at run
// time).  Scale s = fl32(amax / 448); codes E4M3(fl32(x / s)), RNE, saturating at +-448.
#include "fgb_device.hpp"
#include "internal.h"

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
// Floating-Point Arithmetic): with r = RN(1/d) and q0 = RN(x r), the residual x - q0 d is exact in
// one FMA and RN(q0 + residual * r) is the correctly rounded quotient.  Outside the fast range
// the IEEE division is used.  The equality with x / d over every bf16 (x, amax) pair is checked
// exhaustively on the device by fgb_selftest_quotients.
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

// ---------------------------------------------------------------------------------------------
// act_quant: a wave takes one work item at a time (grid-stride), an item being 4 * AQ_UNROLL
// consecutive groups of one token row; 16 lanes per group (16 B = 8 bf16 each), so a wave covers
// 4 groups = 1 KiB of the row per load and issues its AQ_UNROLL loads before any arithmetic.
// Splitting rows into items keeps more waves (and loads) in flight for long rows than one wave per
// row (+10-15% at K = 14336 and 18432).
// ---------------------------------------------------------------------------------------------
constexpr int AQ_THREADS = 512;  // 8 waves (+2-4% over 4 on the large inputs; 16: mixed)
constexpr int AQ_WAVES = AQ_THREADS / 64;
constexpr int AQ_UNROLL = 2;

__global__ __launch_bounds__(AQ_THREADS) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t M, int G, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s_a, int64_t ld_sa) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15, grp = lane >> 4;
  // work item = (token row, chunk of 4 * AQ_UNROLL groups); a wave takes one item at a time
  const int nchunk = (G + 4 * AQ_UNROLL - 1) / (4 * AQ_UNROLL);
  const int64_t items = M * nchunk;
  for (int64_t it = (int64_t)blockIdx.x * AQ_WAVES + (threadIdx.x >> 6); it < items; it += (int64_t)gridDim.x * AQ_WAVES) {
    const int64_t m = it / nchunk;
    const int g0 = (int)(it - m * nchunk) * 4 * AQ_UNROLL;
    const uint16_t* xr = x + m * ldx + sub * 8;
    uint8_t* qr = q + m * ldq + sub * 8;
    uint4 v[AQ_UNROLL];
#pragma unroll
    for (int u = 0; u < AQ_UNROLL; ++u) {
      const int g = g0 + 4 * u + grp;
      v[u] = g < G ? *reinterpret_cast<const uint4*>(xr + g * kBlock) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < AQ_UNROLL; ++u) {
      const int g = g0 + 4 * u + grp;
      const float amax = row16_max(absmax8(v[u]));
      const float s = amax / kE4M3Max;  // IEEE float32 division (correctly rounded)
      const uint2 c = quant8(v[u], make_divisor(s));
      if (g < G) {
        *reinterpret_cast<uint2*>(qr + g * kBlock) = c;
        if (sub == 0) s_a[g * ld_sa + m] = s;
      }
    }
  }
}

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* s_a, int64_t ld_sa, hipStream_t stream) {
  const int G = (int)(K / kBlock);
  const int64_t nchunk = (G + 4 * AQ_UNROLL - 1) / (4 * AQ_UNROLL);
  int64_t blocks = (M * nchunk + AQ_WAVES - 1) / AQ_WAVES;
  if (blocks > 256 * 16) blocks = 256 * 16;  // grid-stride beyond 16 workgroups (128 waves) per CU
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(AQ_THREADS), 0, stream,
                     x, M, G, ldx, q, ldq, s_a, ld_sa);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// weight quant: one 256-thread block per 128x128 block; each thread holds 8 x 16 B (64 values).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void weight_quant_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ wq,
    void* __restrict__ s_w, int fmt) {
  __shared__ float red[4];
  const int64_t KB = K / kBlock;
  const int64_t nb = blockIdx.x / KB, kb = blockIdx.x - (blockIdx.x / KB) * KB;
  const int t = threadIdx.x;
  const int chunk = t & 15;  // 16 B chunk within a 256 B row segment
  const int r0 = t >> 4;     // rows r0, r0+16, ..., r0+112
  uint4 v[8];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t row = nb * kBlock + r0 + 16 * i;
    v[i] = *reinterpret_cast<const uint4*>(w + row * K + kb * kBlock + chunk * 8);
    am = fmaxf(am, absmax8(v[i]));
  }
  am = row16_max(am);
  // across the 4 rows of 16 lanes in a wave, then across waves
  am = fmaxf(am, __shfl_xor(am, 16));
  am = fmaxf(am, __shfl_xor(am, 32));
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s;
  if (fmt == 0) {
    s = am / kE4M3Max;
    if (t == 0) reinterpret_cast<float*>(s_w)[blockIdx.x] = s;
  } else {
    uint32_t code = ue8m0_from_amax(am);
    s = dec_ue8m0(code);
    if (t == 0) reinterpret_cast<uint8_t*>(s_w)[blockIdx.x] = (uint8_t)code;
  }
  const Divisor dv = make_divisor(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t row = nb * kBlock + r0 + 16 * i;
    *reinterpret_cast<uint2*>(wq + row * K + kb * kBlock + chunk * 8) = quant8(v[i], dv);
  }
}

hipError_t launch_weight_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq, void* s_w,
                               int fmt, hipStream_t stream) {
  const int64_t blocks = (N / kBlock) * (K / kBlock);
  hipLaunchKernelGGL(weight_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K,
                     wq, s_w, fmt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// element-wise codecs
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ in,
                                                     uint8_t* __restrict__ out, int64_t n, int fmt,
                                                     int saturate) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    float f = in[i];
    uint32_t c;
    if (fmt == 0) {
      c = cvt_pk_e4m3<false>(f, 0.0f, 0u) & 0xFFu;  // the hardware path used by the quantizers
    } else if (fmt == 1) {
      c = enc_e5m2_int(f, saturate != 0);
    } else {
      c = ue8m0_from_amax(f);
    }
    out[i] = (uint8_t)c;
  }
}

__global__ __launch_bounds__(256) void decode_kernel(const uint8_t* __restrict__ in,
                                                     float* __restrict__ out, int64_t n, int fmt) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    uint32_t c = in[i];
    out[i] = fmt == 0 ? dec_e4m3_int(c) : (fmt == 1 ? dec_e5m2_int(c) : dec_ue8m0(c));
  }
}

// Reference integer E4M3 encoder over an array (checks the hardware conversion).
__global__ __launch_bounds__(256) void encode_e4m3_int_kernel(const float* __restrict__ in,
                                                              uint8_t* __restrict__ out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = (uint8_t)enc_e4m3_sat_int(in[i]);
}

static unsigned ew_blocks(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

hipError_t launch_encode(const float* in, uint8_t* out, int64_t n, int fmt, int saturate,
                         hipStream_t stream) {
  if (fmt == 3) {
    hipLaunchKernelGGL(encode_e4m3_int_kernel, dim3(ew_blocks(n)), dim3(256), 0, stream, in, out, n);
  } else {
    hipLaunchKernelGGL(encode_kernel, dim3(ew_blocks(n)), dim3(256), 0, stream, in, out, n, fmt,
                       saturate);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* in, float* out, int64_t n, int fmt, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3(ew_blocks(n)), dim3(256), 0, stream, in, out, n, fmt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Self-test of the quotient used by the quantizers: for every positive finite bf16 amax and every
// bf16 x with |x| <= amax (both signs), the scale s = fl32(amax/448) and the fast quotient must
// give the same E4M3 code as the IEEE quotient x / s; counts[0] = code mismatches, counts[1] =
// quotients differing in any bit.  One thread per (amax, x) pair of magnitudes.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void selftest_quotients_kernel(unsigned long long* counts) {
  const uint32_t a_bits = blockIdx.y + 1u;          // 0x0001 .. 0x7F7F
  const uint32_t x_bits = blockIdx.x * 256u + threadIdx.x;  // 0x0000 .. 0x7FFF
  unsigned long long code_bad = 0, quot_bad = 0;
  if (x_bits <= a_bits) {
    const float amax = __uint_as_float(a_bits << 16);
    const float s = amax / kE4M3Max;
    const Divisor v = make_divisor(s);
#pragma unroll
    for (int sign = 0; sign < 2; ++sign) {
      const float xv = __uint_as_float((x_bits << 16) | (sign ? 0x80000000u : 0u));
      const float fq = quot(xv, v);
      const float iq = xv / v.d;
      quot_bad += __float_as_uint(fq) != __float_as_uint(iq);
      const uint32_t cf = cvt_pk_e4m3<false>(fq, 0.0f, 0u) & 0xFFu;
      const uint32_t ci = enc_e4m3_sat_int(iq);
      code_bad += cf != ci;
    }
  }
  if (code_bad) atomicAdd(&counts[0], code_bad);
  if (quot_bad) atomicAdd(&counts[1], quot_bad);
}

hipError_t launch_selftest_quotients(unsigned long long* counts, hipStream_t stream) {
  hipLaunchKernelGGL(selftest_quotients_kernel, dim3(0x8000 / 256, 0x7F7F), dim3(256), 0, stream, counts);
  return hipGetLastError();
}

}  // namespace fgb
