// gemm_common.hpp — pieces shared by the block-scaled FP8 GEMM kernels (gfx950).
//
// Matrix-core mapping.  gfx950's v_mfma_f32_16x16x128_f8f6f4 multiplies a 16x128 E4M3 tile by
// a 128x16 E4M3 tile into 16x16 float32: exactly one 128-wide K-block (the activation group and
// weight block edge of Transformers "Fine-grained FP8", intro) per instruction.  The per-block
// product sum P therefore comes out of one instruction, and the block's scales are applied to
// it in registers: acc += P * (s_a[m, kb] * s_w[n/128, kb]).
//
// Operand roles: the weight tile is the MFMA "A" operand (16 output features n) and the
// activation tile the "B" operand (16 tokens m).  Each lane then holds D[n0+4*(lane/16)+r][m0 +
// lane%16], r = 0..3: one token's scale per lane and four consecutive output features, which
// store as one 8-byte bf16 group.
//
// Both operands are loaded with the same K-permutation (lane group g = lane/16 supplies bytes
// 32g .. 32g+31 of the 128-byte K-block row), so the dot product is over the same k for A and B
// whatever the hardware's internal k order within the instruction.
#pragma once
#include "fgb_device.hpp"

namespace fgb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format selects 0/0 = E4M3 for both operands; scale operands 0 select the unscaled opcode
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// The same instruction on E4M3 (CODE 0) or E5M2 (CODE 1) operands, both operands in one format,
// accumulating into c.
template <int CODE>
__device__ __forceinline__ v4f mfma_f8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  static_assert(CODE == 0 || CODE == 1, "E4M3 or E5M2 operands");
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, CODE, CODE, 0, 0, 0, 0);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Global-memory accesses through address-space-1 pointers.  Pointers that reach a kernel inside a
// struct argument are generic to the compiler, which then emits flat instructions; a flat access
// also counts against lgkmcnt, so every later wait for LDS reads would wait for it as well.
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const T __attribute__((address_space(1)))*)p;
}
template <typename T>
__device__ __forceinline__ void gstore(void* p, T v) {
  *(T __attribute__((address_space(1)))*)p = v;
}

__device__ __forceinline__ int4 gload_i4(const void* p) {
  const v4i v = gload<v4i>(p);
  return make_int4(v[0], v[1], v[2], v[3]);
}

// Data read for the last time (weights streamed by the decode kernels) goes with the non-temporal
// hint: the 16-byte load below, and this cache-policy operand of the direct-to-LDS copies.
constexpr int kLastReadAux = 2;
__device__ __forceinline__ int4 gload_i4_last(const void* p) {
  const v4i v = __builtin_nontemporal_load((const v4i __attribute__((address_space(1)))*)p);
  return make_int4(v[0], v[1], v[2], v[3]);
}

// Weight-block scale as float32 from either storage format.
template <int SWF>
__device__ __forceinline__ float load_sw(const void* s_w, int64_t idx) {
  if constexpr (SWF == 0) {
    return gload<float>(reinterpret_cast<const float*>(s_w) + idx);
  } else {
    return dec_ue8m0(gload<uint8_t>(reinterpret_cast<const uint8_t*>(s_w) + idx));
  }
}

// Two float32 values -> two bf16 (round to nearest even) packed in one dword, lo in bits 15:0:
// one v_cvt_pk_bf16_f32 (element-wise casts convert one value per instruction and then need a
// shift and an OR to pack).
typedef float v2f_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_cvt{lo, hi}, v2bf));
}

// Store four consecutive output features of one token.
template <int OUT>
__device__ __forceinline__ void store4(void* y, int64_t ldy, int64_t m, int64_t n, v4f v) {
  if constexpr (OUT == 0) {
    uint16_t* p = reinterpret_cast<uint16_t*>(y) + m * ldy + n;
    v2u w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    gstore<v2u>(p, w);
  } else {
    gstore<v4f>(reinterpret_cast<float*>(y) + m * ldy + n, v);
  }
}

// Workgroup id remapping so that consecutive logical tiles run on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2).  A bijection on [0, nwg).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int per = nwg / 8, rem = nwg % 8;
  const int xcd = bid % 8, local = bid / 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

}  // namespace fgb
