// quant.hip — dynamic activation quantization (1x128 groups), 128x128 weight-block quantization
// and element-wise fp8 codec kernels for gfx950.
//
// Scheme: Transformers "Fine-grained FP8", intro (weights per 128x128 block, activations per
// token per group of 128 along K) and "DeepGEMM fast path" (activation scales computed at run
// time).  Scale s = fl32(amax / 448); codes E4M3(fl32(x / s)), RNE, saturating at +-448.
#include "internal.h"
#include "quant_common.hpp"

namespace fgb {

constexpr float kE5M2Max = 57344.0f;

// Quantize 8 values (4 bf16 pairs) to E5M2 with the IEEE quotient x / d (E5M2 resolves values down
// to 2^-17, where the fast quotient may differ in its last bit) and the integer encoder (RNE,
// saturating at +-57344).
__device__ __forceinline__ uint2 quant8_e5m2(const uint4 w, float d) {
  const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                      bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = enc_e5m2_int(f[i] / d, true);
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// Codes of 8 values for divisor d (the stored scale, or 1 where the scale is 0) in format CODE
// (0 E4M3, 1 E5M2).
template <int CODE>
__device__ __forceinline__ uint2 quant8_code(const uint4 w, float d) {
  if constexpr (CODE == 0) return quant8(w, make_divisor(d));
  else return quant8_e5m2(w, d == 0.0f ? 1.0f : d);
}

// ---------------------------------------------------------------------------------------------
// act_quant: a wave takes one work item at a time (grid-stride), an item being 4 * AQ_UNROLL
// consecutive groups of one token row; 16 lanes per group (16 B = 8 bf16 each), so a wave covers
// 4 groups = 1 KiB of the row per load and issues its AQ_UNROLL loads before any arithmetic.
// Splitting rows into items keeps more waves (and loads) in flight for long rows than one wave per
// row (+10-15% at K = 14336 and 18432).  Inputs and codes are touched once here, so large inputs
// go with the non-temporal hint (+6-15% over default caching on every measured prefill shape,
// e.g. 4096x4096 14.4 -> 12.6 us, 8192x16384 78.6 -> 69.2 us with the 8192-workgroup cap below).
// ---------------------------------------------------------------------------------------------
constexpr int AQ_THREADS = 512;  // 8 waves (+2-4% over 4 on the large inputs; 16: mixed)
constexpr int AQ_WAVES = AQ_THREADS / 64;
constexpr int AQ_UNROLL = 2;
constexpr int64_t AQ_MAX_BLOCKS = 256 * 32;  // grid-stride beyond 32 workgroups per CU

// Inputs of at least this size are streamed with the non-temporal hint (bf16 loads and code
// stores); smaller ones (decode activations, whose codes the GEMM reads right away) keep default
// caching (the fused decode call at 32 x 14336 was 2-4% slower with the hint).
constexpr int64_t kStreamMinBytes = int64_t(16) << 20;

typedef unsigned int aq_u4 __attribute__((ext_vector_type(4)));
typedef unsigned int aq_u2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  if constexpr (NT) {
    const aq_u4 t = __builtin_nontemporal_load(reinterpret_cast<const aq_u4*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ void store8(uint8_t* p, uint2 c) {
  if constexpr (NT) __builtin_nontemporal_store(aq_u2{c.x, c.y}, reinterpret_cast<aq_u2*>(p));
  else *reinterpret_cast<uint2*>(p) = c;
}

template <bool NT>
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
      v[u] = g < G ? load16<NT>(xr + g * kBlock) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < AQ_UNROLL; ++u) {
      const int g = g0 + 4 * u + grp;
      const float amax = row16_max(absmax8(v[u]));
      const float s = amax / kE4M3Max;  // IEEE float32 division (correctly rounded)
      const uint2 c = quant8(v[u], make_divisor(s));
      if (g < G) {
        store8<NT>(qr + g * kBlock, c);
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
  if (blocks > AQ_MAX_BLOCKS) blocks = AQ_MAX_BLOCKS;
  if (M * K * 2 >= kStreamMinBytes)
    hipLaunchKernelGGL(act_quant_kernel<true>, dim3((unsigned)blocks), dim3(AQ_THREADS), 0, stream, x, M, G, ldx, q,
                       ldq, s_a, ld_sa);
  else
    hipLaunchKernelGGL(act_quant_kernel<false>, dim3((unsigned)blocks), dim3(AQ_THREADS), 0, stream, x, M, G, ldx, q,
                       ldq, s_a, ld_sa);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// weight quant: one 256-thread block per 128x128 block; each thread holds 8 x 16 B (64 values).
// ---------------------------------------------------------------------------------------------
template <int CODE>
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
    s = am / (CODE == 0 ? kE4M3Max : kE5M2Max);
    if (t == 0) reinterpret_cast<float*>(s_w)[blockIdx.x] = s;
  } else {
    uint32_t code = ue8m0_from_amax(am);
    s = dec_ue8m0(code);
    if (t == 0) reinterpret_cast<uint8_t*>(s_w)[blockIdx.x] = (uint8_t)code;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t row = nb * kBlock + r0 + 16 * i;
    *reinterpret_cast<uint2*>(wq + row * K + kb * kBlock + chunk * 8) = quant8_code<CODE>(v[i], s);
  }
}

hipError_t launch_weight_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq, void* s_w,
                               int fmt, hipStream_t stream, int code) {
  const int64_t blocks = (N / kBlock) * (K / kBlock);
  if (code == 0)
    hipLaunchKernelGGL(weight_quant_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K, wq, s_w, fmt);
  else
    hipLaunchKernelGGL(weight_quant_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K, wq, s_w, fmt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Per-row quantization: one scale for each whole row (vLLM "FP8 W8A8", "Quantization process":
// per-token activations and per-output-channel weights of the FP8_DYNAMIC scheme).  One
// 256-thread workgroup per row: the amax over the row, s = fl32(amax / max), then the row is read
// again (from the cache) and encoded; that last read and the codes go with the non-temporal hint
// (+7-21% over default caching, 4096x14336 49.7 -> 41.1 us).
// ---------------------------------------------------------------------------------------------
template <int CODE, bool NT>
__global__ __launch_bounds__(256) void row_quant_kernel(const uint16_t* __restrict__ x, int64_t K, int64_t ldx,
                                                        uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s_out) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const int t = threadIdx.x;
  const int nch = (int)(K / 8);  // 16-byte chunks of the row
  const uint16_t* xr = x + m * ldx;
  uint8_t* qr = q + m * ldq;
  float am = 0.0f;
  for (int c = t; c < nch; c += 256) am = fmaxf(am, absmax8(*reinterpret_cast<const uint4*>(xr + 8 * c)));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = am / (CODE == 0 ? kE4M3Max : kE5M2Max);  // IEEE float32 division
  if (t == 0) s_out[m] = s;
  for (int c = t; c < nch; c += 256) store8<NT>(qr + 8 * c, quant8_code<CODE>(load16<NT>(xr + 8 * c), s));
}

hipError_t launch_row_quant(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* s, int code, hipStream_t stream) {
  const bool nt = rows * K * 2 >= kStreamMinBytes;
  if (code == 0 && nt)
    hipLaunchKernelGGL((row_quant_kernel<0, true>), dim3((unsigned)rows), dim3(256), 0, stream, x, K, ldx, q, ldq, s);
  else if (code == 0)
    hipLaunchKernelGGL((row_quant_kernel<0, false>), dim3((unsigned)rows), dim3(256), 0, stream, x, K, ldx, q, ldq, s);
  else if (nt)
    hipLaunchKernelGGL((row_quant_kernel<1, true>), dim3((unsigned)rows), dim3(256), 0, stream, x, K, ldx, q, ldq, s);
  else
    hipLaunchKernelGGL((row_quant_kernel<1, false>), dim3((unsigned)rows), dim3(256), 0, stream, x, K, ldx, q, ldq, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Static quantization with a given per-tensor scale (Transformers "Fine-grained FP8", "DeepGEMM
// fast path": static activations): codes E(fl32(x / s)), s read from device memory.  Grid-stride
// over 16-byte chunks of the rows, two per thread in flight, with the non-temporal hint on the
// input and the codes, up to 32 workgroups per CU (E4M3: 0.65 -> 0.75 of HBM on the large
// inputs, 4096x4096 12.1 -> 10.5 us; E5M2, bound by its IEEE divisions: +8-10%).
// ---------------------------------------------------------------------------------------------
constexpr int SQ_PER_THREAD = 2;
template <int CODE, bool NT>
__global__ __launch_bounds__(256) void static_quant_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                           int64_t ldx, const float* __restrict__ scale,
                                                           uint8_t* __restrict__ q, int64_t ldq) {
  const float s = *scale;
  const int64_t cpr = K / 8, total = M * cpr;
  const int64_t stride = (int64_t)gridDim.x * 256 * SQ_PER_THREAD;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * SQ_PER_THREAD + threadIdx.x; i0 < total; i0 += stride) {
    uint4 v[SQ_PER_THREAD];
#pragma unroll
    for (int u = 0; u < SQ_PER_THREAD; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < total) {
        const int64_t m = i / cpr, c = i - m * cpr;
        v[u] = load16<NT>(x + m * ldx + 8 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < SQ_PER_THREAD; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < total) {
        const int64_t m = i / cpr, c = i - m * cpr;
        store8<NT>(q + m * ldq + 8 * c, quant8_code<CODE>(v[u], s));
      }
    }
  }
}

hipError_t launch_static_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* scale,
                               uint8_t* q, int64_t ldq, int code, hipStream_t stream) {
  int64_t blocks = (M * (K / 8) + 256 * SQ_PER_THREAD - 1) / (256 * SQ_PER_THREAD);
  if (blocks > AQ_MAX_BLOCKS) blocks = AQ_MAX_BLOCKS;
  const bool nt = M * K * 2 >= kStreamMinBytes;
  const dim3 g((unsigned)blocks), b(256);
  if (code == 0 && nt) hipLaunchKernelGGL((static_quant_kernel<0, true>), g, b, 0, stream, x, M, K, ldx, scale, q, ldq);
  else if (code == 0) hipLaunchKernelGGL((static_quant_kernel<0, false>), g, b, 0, stream, x, M, K, ldx, scale, q, ldq);
  else if (nt) hipLaunchKernelGGL((static_quant_kernel<1, true>), g, b, 0, stream, x, M, K, ldx, scale, q, ldq);
  else hipLaunchKernelGGL((static_quant_kernel<1, false>), g, b, 0, stream, x, M, K, ldx, scale, q, ldq);
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
// quotients differing in any bit, counts[2] = those of them whose IEEE quotient has magnitude
// 2^-13 or more.  One thread per (amax, x) pair of magnitudes.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void selftest_quotients_kernel(unsigned long long* counts) {
  const uint32_t a_bits = blockIdx.y + 1u;          // 0x0001 .. 0x7F7F
  const uint32_t x_bits = blockIdx.x * 256u + threadIdx.x;  // 0x0000 .. 0x7FFF
  unsigned long long code_bad = 0, quot_bad = 0, quot_bad_big = 0;
  if (x_bits <= a_bits) {
    const float amax = __uint_as_float(a_bits << 16);
    const float s = amax / kE4M3Max;
    const Divisor v = make_divisor(s);
#pragma unroll
    for (int sign = 0; sign < 2; ++sign) {
      const float xv = __uint_as_float((x_bits << 16) | (sign ? 0x80000000u : 0u));
      const float fq = quot(xv, v);
      const float iq = xv / v.d;
      const bool differ = __float_as_uint(fq) != __float_as_uint(iq);
      quot_bad += differ;
      quot_bad_big += differ && fabsf(iq) >= 0x1p-13f;
      const uint32_t cf = cvt_pk_e4m3<false>(fq, 0.0f, 0u) & 0xFFu;
      const uint32_t ci = enc_e4m3_sat_int(iq);
      code_bad += cf != ci;
    }
  }
  if (code_bad) atomicAdd(&counts[0], code_bad);
  if (quot_bad) atomicAdd(&counts[1], quot_bad);
  if (quot_bad_big) atomicAdd(&counts[2], quot_bad_big);
}

hipError_t launch_selftest_quotients(unsigned long long* counts, hipStream_t stream) {
  hipLaunchKernelGGL(selftest_quotients_kernel, dim3(0x8000 / 256, 0x7F7F), dim3(256), 0, stream, counts);
  return hipGetLastError();
}

}  // namespace fgb
