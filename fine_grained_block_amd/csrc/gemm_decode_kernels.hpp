// gemm_decode_kernels.hpp — the decode (M <= 64) block-scaled FP8 GEMM kernels; included by
// the translation units that instantiate and launch them.
//
// Same result as the prefill path (Transformers "Fine-grained FP8", "DeepGEMM fast path"), but
// for few tokens the weight stream dominates (bytes per weight: 1 for FP8, per the Baseten
// NVFP4 summary, "Less memory, more compute"), so the kernels are organised to keep HBM busy:
//   * M <= 16: one workgroup per 16 weight rows and the whole K, its waves splitting the
//     K-blocks; weights >= 48 MiB with K >= 8192 stream through per-wave LDS rings with
//     whole-line direct copies, the others load whole lines into registers and reorder them
//     through LDS.  One launch.
//   * 16 < M <= 64, weights of at most 16 MiB: the per-wave ring kernel with 32 or 64 activation
//     rows, one launch.
//   * 16 < M <= 64, larger weights: a workgroup of 2, 4 or 8 waves (16 weight rows each) over a
//     K slice, weights, activations and their scales streamed through an LDS ring shared by the
//     waves; 8-wave workgroups (one 128-row weight block) slice K only to occupy the CUs, and
//     sliced shapes add their float32 partials [S][M][N] in a second, ordered launch; with at
//     most 32 activation rows and 32-63 K-blocks, 2- or 4-wave workgroups cover the weight rows
//     over the whole K in one launch.  (A reduction inside the same launch costs more on
//     this multi-XCD part, whose L2s are not coherent with each other: with release fences the L2
//     is written back; with the partials stored and loaded at device scope past the L2 and a
//     counter electing the last slice, 1.7-2.4x slower than the second launch.)
//   * MoE with at most 64 rows per expert: the M <= 16 register kernel per (16 weight rows,
//     expert), walking the expert's rows in passes of 16 or 32.
//   * From bf16 activations, a few tokens: the per-wave ring kernel that quantizes each 1x128
//     group itself before its MFMA.
// Weight rows read for the last time are loaded with the non-temporal hint (streamed from HBM:
// +3-11% at M <= 16, +2-8% at 17-32 rows); not in the 64-row shared-ring kernel, where the hint
// measured up to 5% slower on 3 of 5 shapes, nor in MoE passes whose rows are read again.
#pragma once
#include <type_traits>

#include "gemm_common.hpp"
#include "internal.h"
#include "quant_common.hpp"

namespace fgb {

namespace {


// 16-byte chunk c of LDS row r sits at c ^ ((r & 7) ^ (r>>3 & 1)): conflict-free 16-row fragment
// reads on gfx950's 64-bank LDS.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

// Sum of the S partial slices in slice order; all loads of a group of 8 slices are issued
// before they are added.  SCH 1 and 2 (scales that do not vary along K, see the ring kernel)
// then multiply by the token's or the tensor's activation scale s_a (a_kind 1 or 2) and, for
// SCH 2, by the channels' weight scales s_w[n .. n+3].
template <int OUT, int SCH = 0>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int S, int64_t M,
                                                            int64_t N, void* y, int64_t ldy, const float* s_a,
                                                            int a_kind, const float* s_w) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one float4 of y
  const int64_t total = M * (N / 4);
  if (q >= total) return;
  const int64_t m = q / (N / 4), n = (q - m * (N / 4)) * 4;
  const float* base = ws + m * N + n;
  const int64_t slice = M * N;
  v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i0 = 0; i0 < S; i0 += 8) {
    v4f v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = i0 + u < S ? gload<v4f>(base + (int64_t)(i0 + u) * slice) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u < S) s += v[u];
    }
  }
  if constexpr (SCH != 0) {
    s = s * gload<float>(s_a + (a_kind == 2 ? 0 : m));
    if constexpr (SCH == 2) s = s * gload<v4f>(s_w + n);
  }
  store4<OUT>(y, ldy, m, n, s);
}

#define GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int V>
constexpr int vmcnt_only() { return (V & 0xF) | ((V >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// gfx950 LDS: 16-byte chunk c of 128-byte row r at c ^ ((r & 7) ^ (r>>3 & 1))
__device__ __forceinline__ int swz_g(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// ---------------------------------------------------------------------------------------------
// Weight-streaming kernel with per-wave LDS rings.  A workgroup owns 16 weight rows and the whole
// K; its WK waves split the K-blocks into contiguous slices and add their partial tiles through
// LDS at the end (one launch, no workspace).  Each wave streams its 16 weight rows, the MR
// activation rows of its slice (rows >= M repeat row M-1; their results are dropped) and their
// scales through a private ring of D LDS stages with whole-line direct copies.  A copy instruction
// reads 8 whole 128-byte lines, where loading the MFMA operand layout straight into registers
// touches 16 half-used lines per instruction, which costs about four times as much address-unit
// time per byte on gfx950.  No barrier is needed until the partial tiles are added.  MR = 32 or
// 64 gives each wave MR/16 token tiles, all multiplied by the same weight fragment.
//
// SCH and CODE as for the prefill kernel: 0 = per-group activation and per-block weight scales;
// 1 = per-block weight scales, the per-token or per-tensor activation scale in the epilogue; 2 =
// per-channel weight scales and per-token or per-tensor activation scales, both in the epilogue
// (the MFMAs accumulate in place).  CODE 1: E5M2 operands (schemes 1 and 2).
//
template <int WK, int MR, int D, int SWF, int OUT, int SCH = 0, int CODE = 0>
__global__ __launch_bounds__(64 * WK) void gemm_decode_ring_kernel(GemmArgs p) {
  static_assert(SCH != 0 || CODE == 0, "the 1x128-group scheme runs on E4M3 operands");
  constexpr int MT = MR >= 16 ? MR / 16 : 1;  // token tiles per wave
  constexpr int WST = 16 * 128, AST = MR * 128, SST = 64 * 4;
  constexpr int STAGE = WST + AST + SST;
  constexpr int OPS = 2 + MR / 8 + (SCH == 0 ? 1 : 0);  // direct copies per stage
  static_assert(MR == 8 || MR == 16 || MR == 32 || MR == 64, "8, 16, 32 or 64 activation rows");
  static_assert((D - 1) * OPS <= 63, "copies in flight fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[WK * D * STAGE];
  __shared__ v4f red[WK > 1 ? WK - 1 : 1][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = p.K;
  const int64_t M = p.M;
  const int KB = (int)(K / 128);
  const int per = (KB + WK - 1) / WK;
  const int kb0 = min(KB, wave * per);
  const int nk = min(KB, kb0 + per) - kb0;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nb = n0 / 128;
  uint8_t* const wring = ring + wave * D * STAGE;

  // weight-block scales of this wave's slice, lane l holding block kb0 + l + 64 t (K <= 32768)
  float sw0 = 0.0f, sw1 = 0.0f, sw2 = 0.0f, sw3 = 0.0f;
  if constexpr (SCH != 2) {
    const int64_t b = nb * KB + kb0;
    sw0 = lane < nk ? load_sw<SWF>(p.s_w, b + lane) : 0.0f;
    sw1 = lane + 64 < nk ? load_sw<SWF>(p.s_w, b + lane + 64) : 0.0f;
    sw2 = lane + 128 < nk ? load_sw<SWF>(p.s_w, b + lane + 128) : 0.0f;
    sw3 = lane + 192 < nk ? load_sw<SWF>(p.s_w, b + lane + 192) : 0.0f;
  }
  auto sw_at = [&](int kk) -> float {
    const int l = kk & 63, t = kk >> 6;
    const int r0 = __builtin_amdgcn_readlane(__float_as_int(sw0), l);
    const int r1 = __builtin_amdgcn_readlane(__float_as_int(sw1), l);
    const int r2 = __builtin_amdgcn_readlane(__float_as_int(sw2), l);
    const int r3 = __builtin_amdgcn_readlane(__float_as_int(sw3), l);
    const int lo = (t & 1) ? r1 : r0, hi = (t & 1) ? r3 : r2;
    return __int_as_float((t & 2) ? hi : lo);
  };

  // copy sources: lane i of 8-row group q takes row 8q + i/8, logical chunk (i%8) ^ g(row)
  uint32_t woff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * q + (lane >> 3);
    woff[q] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint8_t* wbase = p.w_q + n0 * K;

  uint32_t aoff[MR / 8];
#pragma unroll
  for (int q = 0; q < MR / 8; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int64_t m = r < M ? r : M - 1;
    aoff[q] = (uint32_t)(m * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint32_t soff = (uint32_t)((lane < M ? lane : M - 1) * 4);

  // 8-row activation copy groups that hold real rows (the others would only repeat row M-1 into
  // rows whose outputs are not stored): fewer copies where M is below the staged rows
  const int agrp = (int)min((int64_t)(MR / 8), (M + 7) / 8);
  auto issue = [&](int kk) {
    uint8_t* st = wring + (kk % D) * STAGE;
    const int64_t kb = kb0 + kk;
    const uint8_t* wb = wbase + kb * 128;
    const uint8_t* ab = p.a_q + kb * 128;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(p.s_a + kb * p.ld_sa);
    asm volatile("" : "+s"(wb));
    asm volatile("" : "+s"(ab));
    asm volatile("" : "+s"(sb));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t o = woff[q];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(GPTR(wb + o), LPTR(st + q * 1024), 16, 0, kLastReadAux);
    }
#pragma unroll
    for (int q = 0; q < MR / 8; ++q) {
      if (q < agrp) {
        uint32_t o = aoff[q];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds(GPTR(ab + o), LPTR(st + WST + q * 1024), 16, 0, 0);
      }
    }
    if constexpr (SCH == 0) {
      uint32_t o = soff;
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(GPTR(sb + o), LPTR(st + WST + AST), 4, 0, 0);
    }
  };

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(min(i, nk - 1));
    for (int kk = 0; kk < nk; ++kk) {
      // refill the stage consumed one block ago (clamped past the slice: never a pending stage)
      issue(min(kk + D - 1, nk - 1));
      // own copies of this block landed, the D-1 younger stages' may stay in flight
      // (2 + agrp + 1 copies per stage; the wait count is an immediate, hence the cases)
      {
        constexpr int FIX = OPS - MR / 8;
        if (agrp == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + 1)>());
        else if (agrp == 2) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 16 ? 2 : 1))>());
        else if (agrp == 3) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 32 ? 3 : 1))>());
        else if (agrp == 4) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 32 ? 4 : 1))>());
        else if (agrp == 5) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 64 ? 5 : 1))>());
        else if (agrp == 6) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 64 ? 6 : 1))>());
        else if (agrp == 7) __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * (FIX + (MR >= 64 ? 7 : 1))>());
        else __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * OPS>());
      }
      // The LDS reads are written as one asm block that also waits for them: the compiler cannot
      // tell this wave's ring stages apart and would otherwise wait for every copy in flight.
      const uint32_t st = (uint32_t)(uintptr_t)LPTR(wring + (kk % D) * STAGE);
      const int r = lane & 15, g = lane >> 4;
      const uint32_t aw0 = st + swz(r, 2 * g), aw1 = st + swz(r, 2 * g + 1);
      const int ra = r & (MR - 1);
      const uint32_t aa0 = st + WST + swz(ra, 2 * g), aa1 = st + WST + swz(ra, 2 * g + 1);
      const uint32_t as = st + WST + AST + 4 * r;
      v4i w0, w1, a0[MT], a1[MT];
      float sa[MT];
      if constexpr (MT == 1) {
        asm volatile(
            "ds_read_b128 %0, %5\n\t"
            "ds_read_b128 %1, %6\n\t"
            "ds_read_b128 %2, %7\n\t"
            "ds_read_b128 %3, %8\n\t"
            "ds_read_b32 %4, %9\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1), "=&v"(a0[0]), "=&v"(a1[0]), "=&v"(sa[0])
            : "v"(aw0), "v"(aw1), "v"(aa0), "v"(aa1), "v"(as)
            : "memory");
      } else if constexpr (MT == 2) {
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %9\n\t"
            "ds_read_b128 %2, %10\n\t"
            "ds_read_b128 %3, %11\n\t"
            "ds_read_b128 %4, %10 offset:2048\n\t"
            "ds_read_b128 %5, %11 offset:2048\n\t"
            "ds_read_b32 %6, %12\n\t"
            "ds_read_b32 %7, %12 offset:64\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1), "=&v"(a0[0]), "=&v"(a1[0]), "=&v"(a0[1]), "=&v"(a1[1]), "=&v"(sa[0]),
              "=&v"(sa[1])
            : "v"(aw0), "v"(aw1), "v"(aa0), "v"(aa1), "v"(as)
            : "memory");
      } else {
        asm volatile(
            "ds_read_b128 %0, %14\n\t"
            "ds_read_b128 %1, %15\n\t"
            "ds_read_b128 %2, %16\n\t"
            "ds_read_b128 %3, %17\n\t"
            "ds_read_b128 %4, %16 offset:2048\n\t"
            "ds_read_b128 %5, %17 offset:2048\n\t"
            "ds_read_b128 %6, %16 offset:4096\n\t"
            "ds_read_b128 %7, %17 offset:4096\n\t"
            "ds_read_b128 %8, %16 offset:6144\n\t"
            "ds_read_b128 %9, %17 offset:6144\n\t"
            "ds_read_b32 %10, %18\n\t"
            "ds_read_b32 %11, %18 offset:64\n\t"
            "ds_read_b32 %12, %18 offset:128\n\t"
            "ds_read_b32 %13, %18 offset:192\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(w0), "=&v"(w1), "=&v"(a0[0]), "=&v"(a1[0]), "=&v"(a0[1]), "=&v"(a1[1]), "=&v"(a0[2]),
              "=&v"(a1[2]), "=&v"(a0[3]), "=&v"(a1[3]), "=&v"(sa[0]), "=&v"(sa[1]), "=&v"(sa[2]), "=&v"(sa[3])
            : "v"(aw0), "v"(aw1), "v"(aa0), "v"(aa1), "v"(as)
            : "memory");
      }
      v8i wf;
      wf[0] = w0[0]; wf[1] = w0[1]; wf[2] = w0[2]; wf[3] = w0[3];
      wf[4] = w1[0]; wf[5] = w1[1]; wf[6] = w1[2]; wf[7] = w1[3];
      // (schemes 1 and 2 copy no activation scales: their sa reads see stale bytes, unused)
      const float sw = SCH == 2 ? 0.0f : sw_at(kk);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        v8i af;
        af[0] = a0[j][0]; af[1] = a0[j][1]; af[2] = a0[j][2]; af[3] = a0[j][3];
        af[4] = a1[j][0]; af[5] = a1[j][1]; af[6] = a1[j][2]; af[7] = a1[j][3];
        if constexpr (SCH == 0) acc[j] += mfma_e4m3_16x16x128(wf, af) * (sa[j] * sw);
        else if constexpr (SCH == 1) acc[j] += mfma_f8_16x16x128<CODE>(wf, af, v4f{0.0f, 0.0f, 0.0f, 0.0f}) * sw;
        else acc[j] = mfma_f8_16x16x128<CODE>(wf, af, acc[j]);
      }
    }
  }
  // the clamped copies past the slice must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
  auto store_rows = [&]() {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int m = 16 * j + (lane & 15);
      if (m < M) {
        if constexpr (SCH != 0) {
          // scales that do not vary along K: the token's (or the tensor's), then the channels'
          acc[j] = acc[j] * gload<float>(p.s_a + (p.a_kind == 2 ? 0 : m));
          if constexpr (SCH == 2) acc[j] = acc[j] * gload<v4f>(reinterpret_cast<const float*>(p.s_w) + n0 + 4 * (lane >> 4));
        }
        store4<OUT>(p.y, p.ldy, m, n0 + 4 * (lane >> 4), acc[j]);
      }
    }
  };
  if constexpr (WK > 1) {
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < MT; ++j) red[wave - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[j] += red[w][j][lane];
  }
  store_rows();
}

// ---------------------------------------------------------------------------------------------
// The weight streaming of the ring kernel with the dynamic activation quantization done in the
// kernel, for M <= 8 (Transformers "Fine-grained FP8", intro and "DeepGEMM fast path":
// activation scales computed at run time per token and 1x128 group).  Each wave streams its 16
// weight rows and the bf16 activation rows of its K-slice through its ring and quantizes every
// 128-element group right before its MFMA with the quantizer's own arithmetic (s = fl32(amax /
// 448), codes E4M3(fl32(x / s))), so codes and scales equal those of act_quant and, with the
// two-launch path's K split and summation order, so does the float32 result.  Only the MQ (>= M,
// a power of two up to 8) real rows are quantized, spread over all 64 lanes (2*MQ elements per
// lane, 64/MQ lanes per row).  The bf16 rows are 256 bytes in LDS, 16-byte chunk c of row r at
// c ^ (r & 15).  The codes and the row scales go to a per-wave LDS tile in the MFMA operand
// layout (16 rows of 128 bytes, rows >= MQ never written: they feed only output columns of
// tokens >= M, which are not stored), from which the B operand is read as in the ring kernel.
template <int WK, int MQ, int D, int SWF, int OUT>
__global__ __launch_bounds__(64 * WK) void gemm_decode_fused_quant_small_kernel(GemmArgs p,
                                                                                const uint16_t* __restrict__ x,
                                                                                int64_t ldx) {
  static_assert(MQ == 1 || MQ == 2 || MQ == 4 || MQ == 8, "1, 2, 4 or 8 quantized rows");
  constexpr int MRC = MQ < 4 ? 4 : MQ;            // staged bf16 rows (copies move 4 rows at a time)
  constexpr int WST = 16 * 128, AST = MRC * 256;
  constexpr int STAGE = WST + AST;
  constexpr int OPS = 2 + MRC / 4;
  constexpr int E = 2 * MQ;                        // elements per lane
  constexpr int LPR = 64 / MQ;                     // lanes per row
  static_assert((D - 1) * OPS <= 63, "copies in flight fit the vmcnt counter");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[WK * D * STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ctile[WK][16 * 128];  // codes, MFMA B layout
  __shared__ float stile[WK][16];                                         // row scales
  __shared__ v4f red[WK > 1 ? WK - 1 : 1][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = p.K, M = p.M;
  const int KB = (int)(K / 128);
  const int per = (KB + WK - 1) / WK;
  const int kb0 = min(KB, wave * per);
  const int nk = min(KB, kb0 + per) - kb0;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nb = n0 / 128;
  uint8_t* const wring = ring + wave * D * STAGE;

  uint32_t woff[2], aoff[MRC / 4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * q + (lane >> 3);
    woff[q] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
#pragma unroll
  for (int q = 0; q < MRC / 4; ++q) {
    const int r = 4 * q + (lane >> 4);
    const int64_t m = r < M ? r : M - 1;
    aoff[q] = (uint32_t)(m * ldx * 2 + (((lane & 15) ^ (r & 15)) * 16));
  }
  const uint8_t* wbase = p.w_q + n0 * K;

  auto issue = [&](int kk) {
    uint8_t* st = wring + (kk % D) * STAGE;
    const int64_t kb = kb0 + kk;
    const uint8_t* wb = wbase + kb * 128;
    const uint8_t* ab = reinterpret_cast<const uint8_t*>(x) + kb * 256;
    asm volatile("" : "+s"(wb));
    asm volatile("" : "+s"(ab));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t o = woff[q];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(GPTR(wb + o), LPTR(st + q * 1024), 16, 0, kLastReadAux);
    }
#pragma unroll
    for (int q = 0; q < MRC / 4; ++q) {
      uint32_t o = aoff[q];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(GPTR(ab + o), LPTR(st + WST + q * 1024), 16, 0, 0);
    }
  };

  float sw0 = 0.0f, sw1 = 0.0f, sw2 = 0.0f, sw3 = 0.0f;
  {
    const int64_t b = nb * KB + kb0;
    sw0 = lane < nk ? load_sw<SWF>(p.s_w, b + lane) : 0.0f;
    sw1 = lane + 64 < nk ? load_sw<SWF>(p.s_w, b + lane + 64) : 0.0f;
    sw2 = lane + 128 < nk ? load_sw<SWF>(p.s_w, b + lane + 128) : 0.0f;
    sw3 = lane + 192 < nk ? load_sw<SWF>(p.s_w, b + lane + 192) : 0.0f;
  }
  auto sw_at = [&](int kk) -> float {
    const int l = kk & 63, t = kk >> 6;
    const int r0 = __builtin_amdgcn_readlane(__float_as_int(sw0), l);
    const int r1 = __builtin_amdgcn_readlane(__float_as_int(sw1), l);
    const int r2 = __builtin_amdgcn_readlane(__float_as_int(sw2), l);
    const int r3 = __builtin_amdgcn_readlane(__float_as_int(sw3), l);
    const int lo = (t & 1) ? r1 : r0, hi = (t & 1) ? r3 : r2;
    return __int_as_float((t & 2) ? hi : lo);
  };

  // this lane's share of the quantization: row rq, elements eo .. eo + E - 1 of the group
  const int rq = lane / LPR, eo = (lane % LPR) * E;
  const uint32_t xsrc = (uint32_t)(WST + rq * 256 + ((((eo * 2) >> 4) ^ (rq & 15)) << 4) + ((eo * 2) & 15));
  const uint32_t cdst = (uint32_t)(uintptr_t)LPTR(&ctile[wave][0]) + rq * 128 + ((((eo >> 4)) ^ swz_g(rq)) << 4) + (eo & 15);
  const int r = lane & 15, g = lane >> 4;
  const uint32_t cb0 = (uint32_t)(uintptr_t)LPTR(&ctile[wave][0]) + swz(r, 2 * g);
  const uint32_t cb1 = (uint32_t)(uintptr_t)LPTR(&ctile[wave][0]) + swz(r, 2 * g + 1);
  const uint32_t sdst = (uint32_t)(uintptr_t)LPTR(&stile[wave][rq]);
  const uint32_t ssrc = (uint32_t)(uintptr_t)LPTR(&stile[wave][r]);

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(min(i, nk - 1));
    for (int kk = 0; kk < nk; ++kk) {
      issue(min(kk + D - 1, nk - 1));
      __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * OPS>());
      const uint32_t st = (uint32_t)(uintptr_t)LPTR(wring + (kk % D) * STAGE);
      // this lane's E bf16 values (one LDS read; E = 16 is two 16-byte chunks)
      uint32_t xv[E / 2];
      if constexpr (E == 2) {
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(xv[0]) : "v"(st + xsrc) : "memory");
      } else if constexpr (E == 4) {
        v2u t;
        asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(t) : "v"(st + xsrc) : "memory");
        xv[0] = t[0]; xv[1] = t[1];
      } else if constexpr (E == 8) {
        v4i t;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(t) : "v"(st + xsrc) : "memory");
        xv[0] = t[0]; xv[1] = t[1]; xv[2] = t[2]; xv[3] = t[3];
      } else {
        // 16 elements = logical chunks 2c and 2c+1 of the row, each at its own swizzled slot
        const int c = eo >> 3;
        const uint32_t a0 = st + WST + rq * 256 + (((c) ^ (rq & 15)) << 4);
        const uint32_t a1 = st + WST + rq * 256 + (((c + 1) ^ (rq & 15)) << 4);
        v4i t0, t1;
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(t0), "=&v"(t1) : "v"(a0), "v"(a1) : "memory");
        xv[0] = t0[0]; xv[1] = t0[1]; xv[2] = t0[2]; xv[3] = t0[3];
        xv[4] = t1[0]; xv[5] = t1[1]; xv[6] = t1[2]; xv[7] = t1[3];
      }
      float f[E];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        f[2 * i] = bf16_lo(xv[i]);
        f[2 * i + 1] = bf16_hi(xv[i]);
      }
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) am = fmaxf(am, fabsf(f[i]));
      am = group_max_nonneg<LPR>(am);
      const float sa = am / kE4M3Max;  // IEEE float32 division, as act_quant
      const Divisor dv = make_divisor(sa);
      if (__all(dv.fast)) {
#pragma unroll
        for (int i = 0; i < E; ++i) f[i] = quot_fast(f[i], dv);
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) f[i] = quot(f[i], dv);
      }
      uint32_t cw[E / 4 > 0 ? E / 4 : 1];
      if constexpr (E == 2) {
        cw[0] = cvt_pk_e4m3<false>(f[0], f[1], 0u) & 0xFFFFu;
        asm volatile("ds_write_b16 %0, %1" ::"v"(cdst), "v"(cw[0]) : "memory");
      } else {
#pragma unroll
        for (int i = 0; i < E / 4; ++i) cw[i] = cvt_pk_e4m3<true>(f[4 * i + 2], f[4 * i + 3], cvt_pk_e4m3<false>(f[4 * i], f[4 * i + 1], 0u));
        if constexpr (E == 4) {
          asm volatile("ds_write_b32 %0, %1" ::"v"(cdst), "v"(cw[0]) : "memory");
        } else if constexpr (E == 8) {
          v2u t = {cw[0], cw[1]};
          asm volatile("ds_write_b64 %0, %1" ::"v"(cdst), "v"(t) : "memory");
        } else {
          v4i t = {(int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3]};
          asm volatile("ds_write_b128 %0, %1" ::"v"(cdst), "v"(t) : "memory");
        }
      }
      if (lane % LPR == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(sdst), "v"(sa) : "memory");
      // the wave's own writes are done before it reads the tile back (LDS serves a wave in order)
      v4i w0, w1, b0, b1;
      float sar;
      const uint32_t aw0 = st + swz(r, 2 * g), aw1 = st + swz(r, 2 * g + 1);
      asm volatile(
          "s_waitcnt lgkmcnt(0)\n\t"
          "ds_read_b128 %0, %5\n\t"
          "ds_read_b128 %1, %6\n\t"
          "ds_read_b128 %2, %7\n\t"
          "ds_read_b128 %3, %8\n\t"
          "ds_read_b32 %4, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(w0), "=&v"(w1), "=&v"(b0), "=&v"(b1), "=&v"(sar)
          : "v"(aw0), "v"(aw1), "v"(cb0), "v"(cb1), "v"(ssrc)
          : "memory");
      v8i wf, af;
      wf[0] = w0[0]; wf[1] = w0[1]; wf[2] = w0[2]; wf[3] = w0[3];
      wf[4] = w1[0]; wf[5] = w1[1]; wf[6] = w1[2]; wf[7] = w1[3];
      af[0] = b0[0]; af[1] = b0[1]; af[2] = b0[2]; af[3] = b0[3];
      af[4] = b1[0]; af[5] = b1[1]; af[6] = b1[2]; af[7] = b1[3];
      acc += mfma_e4m3_16x16x128(wf, af) * (sar * sw_at(kk));
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
  if constexpr (WK > 1) {
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) acc += red[w][lane];
  }
  if ((lane & 15) < M) store4<OUT>(p.y, p.ldy, lane & 15, n0 + 4 * (lane >> 4), acc);
}

// ---------------------------------------------------------------------------------------------
// 16 < M <= 128: a workgroup of NW waves owns 16*NW weight rows (16 per wave; 8 waves: one 128-row
// weight block) over a slice of K-blocks.  The rows, the 16*MT activation rows (rows >= M repeat
// row M-1; their results are dropped) and the activation scales of each K-block stream through a
// ring of D LDS stages shared by the waves, with whole-line buffer-form direct copies issued D-1
// blocks ahead and one barrier per block; the activation stream is read once per 16*NW weight
// rows.  Slices (S > 1) write float32 partials [S][M][N] for the ordered reduction launch.
// SCH and CODE as for the ring kernel (schemes 1 and 2 copy no activation scales; their scales
// that do not vary along K multiply the finished sums, here or in the reduction).
// ---------------------------------------------------------------------------------------------
template <int NW, int MT, int D, int SWF, int OUT, int SCH = 0, int CODE = 0>
__global__ __launch_bounds__(64 * NW, 1) void gemm_decode_mid_kernel(GemmArgs p, int kpw, int S, float* ws) {
  static_assert(SCH != 0 || CODE == 0, "the 1x128-group scheme runs on E4M3 operands");
  static_assert(NW == 2 || NW == 4 || NW == 8, "2, 4 or 8 waves");
  constexpr int MROWS = 16 * MT;
  constexpr int WB = 16 * NW * 128, AB = MROWS * 128, SB = (MT == 8 ? 128 : 64) * 4;
  constexpr int STAGE = WB + AB + SB;
  constexpr int A_GRP = MROWS / 8;                      // 8-row copy groups of the activation rows
  constexpr int A_PER = A_GRP >= NW ? A_GRP / NW : 1;   // activation copies per wave per block
  constexpr int SA_CP = MT == 8 ? 2 : 1;                // 64-token copies of the activation scales
  constexpr int OPS = 2 + A_PER + (SCH == 0 ? SA_CP : 0);  // copies per wave per block: W, A, scales
  static_assert(D >= 3 && (D - 2) * OPS <= 63, "three or more stages, in-flight copies within vmcnt");
  static_assert(MT == 2 || MT == 4 || MT == 8, "32, 64 or 128 activation rows");
  static_assert(MT != 8 || NW == 8, "128 activation rows: 8 waves");
  static_assert(D * STAGE + 1024 <= 160 * 1024, "the ring fits in LDS");
  // one array: the stages' LDS reads are asm blocks that wait for themselves (below), so the
  // compiler need not tell the stages apart
  __shared__ __attribute__((aligned(1024))) uint8_t ring[D * STAGE];
  __shared__ float sws[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = p.K, N = p.N, M = p.M;
  const int KB = (int)(K / 128);
  const int nt = blockIdx.x / S, split = blockIdx.x - nt * S;
  const int kb0 = split * kpw;
  const int nk = min(KB, kb0 + kpw) - kb0;
  const int64_t n0 = (int64_t)nt * 16 * NW;

  // copy sources: lane i of 8-row group q takes row 8q + i/8, logical chunk (i%8) ^ g(row); with
  // more waves than activation groups, waves repeat earlier groups (same bytes to the same place)
  uint32_t woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (wave + NW * i) + (lane >> 3);
    woff[i] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
  int agrp[A_PER];
  uint32_t aoff[A_PER];
#pragma unroll
  for (int j = 0; j < A_PER; ++j) {
    agrp[j] = A_GRP >= NW ? wave + NW * j : wave % A_GRP;
    const int r = 8 * agrp[j] + (lane >> 3);
    const int64_t m = r < M ? r : M - 1;
    aoff[j] = (uint32_t)(m * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint32_t soff = (uint32_t)((lane < M ? lane : M - 1) * 4);
  const uint32_t soff2 = (uint32_t)((lane + 64 < M ? lane + 64 : M - 1) * 4);  // tokens 64..127

  auto issue = [&](int kk, uint8_t* st) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the builtins exist in the device pass only)
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_q + n0 * K), 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.s_a, 0, -1, 0x00020000);
    const int kb = kb0 + kk;
    const uint32_t koff = (uint32_t)kb * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, LPTR(st + (wave + NW * i) * 1024), 16, woff[i], koff, 0,
                                               MT == 2 ? kLastReadAux : 0);
#pragma unroll
    for (int j = 0; j < A_PER; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, LPTR(st + WB + agrp[j] * 1024), 16, aoff[j], koff, 0, 0);
    if constexpr (SCH == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rs, LPTR(st + WB + AB), 4, soff, (uint32_t)(kb * p.ld_sa * 4), 0, 0);
      if constexpr (MT == 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rs, LPTR(st + WB + AB + 256), 4, soff2, (uint32_t)(kb * p.ld_sa * 4),
                                                 0, 0);
    }
#endif
  };
  auto stage = [&](int i) -> uint8_t* { return ring + i * STAGE; };

  if constexpr (SCH != 2) {
    for (int c = tid; c < nk; c += 64 * NW) sws[c] = load_sw<SWF>(p.s_w, (n0 / 128) * KB + kb0 + c);
    // own LDS writes complete before the first step's barrier, which has no fence: LDS
    // operations of different waves may be served out of order
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  }

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int r = lane & 15, g = lane >> 4;
  auto step = [&](int kk, const uint8_t* cur, uint8_t* refill) {
    // own copies of block kk landed (the younger D-2 blocks' stay in flight), then everyone's:
    // an execution barrier only (__syncthreads' fence would wait for every copy in flight)
    __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 2) * OPS>());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(kk + D - 1, nk - 1), refill);  // into the stage consumed one block ago
    // The stage's LDS reads are one asm block that also waits for them: after the step guards
    // below (control-flow joins) the compiler can no longer tell the ring stages apart and would
    // wait for every copy in flight.
    const uint32_t b = (uint32_t)(uintptr_t)LPTR(cur);
    const uint32_t w0 = b + swz(16 * wave + r, 2 * g), w1 = b + swz(16 * wave + r, 2 * g + 1);
    const uint32_t a0 = b + WB + swz(r, 2 * g), a1 = b + WB + swz(r, 2 * g + 1);
    const uint32_t sp = b + WB + AB + 4 * r;
    v4i wl, wh, al[MT], ah[MT];
    float sa[MT];
    if constexpr (MT == 2) {
      asm volatile(
          "ds_read_b128 %0, %8\n\t"
          "ds_read_b128 %1, %9\n\t"
          "ds_read_b128 %2, %10\n\t"
          "ds_read_b128 %3, %11\n\t"
          "ds_read_b128 %4, %10 offset:2048\n\t"
          "ds_read_b128 %5, %11 offset:2048\n\t"
          "ds_read_b32 %6, %12\n\t"
          "ds_read_b32 %7, %12 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(wl), "=&v"(wh), "=&v"(al[0]), "=&v"(ah[0]), "=&v"(al[1]), "=&v"(ah[1]), "=&v"(sa[0]), "=&v"(sa[1])
          : "v"(w0), "v"(w1), "v"(a0), "v"(a1), "v"(sp)
          : "memory");
    } else {
      // (MT == 8: token tiles 4..7 follow in a second block)
      asm volatile(
          "ds_read_b128 %0, %14\n\t"
          "ds_read_b128 %1, %15\n\t"
          "ds_read_b128 %2, %16\n\t"
          "ds_read_b128 %3, %17\n\t"
          "ds_read_b128 %4, %16 offset:2048\n\t"
          "ds_read_b128 %5, %17 offset:2048\n\t"
          "ds_read_b128 %6, %16 offset:4096\n\t"
          "ds_read_b128 %7, %17 offset:4096\n\t"
          "ds_read_b128 %8, %16 offset:6144\n\t"
          "ds_read_b128 %9, %17 offset:6144\n\t"
          "ds_read_b32 %10, %18\n\t"
          "ds_read_b32 %11, %18 offset:64\n\t"
          "ds_read_b32 %12, %18 offset:128\n\t"
          "ds_read_b32 %13, %18 offset:192\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(wl), "=&v"(wh), "=&v"(al[0]), "=&v"(ah[0]), "=&v"(al[1]), "=&v"(ah[1]), "=&v"(al[2]),
            "=&v"(ah[2]), "=&v"(al[3]), "=&v"(ah[3]), "=&v"(sa[0]), "=&v"(sa[1]), "=&v"(sa[2]), "=&v"(sa[3])
          : "v"(w0), "v"(w1), "v"(a0), "v"(a1), "v"(sp)
          : "memory");
      if constexpr (MT == 8) {
        asm volatile(
            "ds_read_b128 %0, %12 offset:8192\n\t"
            "ds_read_b128 %1, %13 offset:8192\n\t"
            "ds_read_b128 %2, %12 offset:10240\n\t"
            "ds_read_b128 %3, %13 offset:10240\n\t"
            "ds_read_b128 %4, %12 offset:12288\n\t"
            "ds_read_b128 %5, %13 offset:12288\n\t"
            "ds_read_b128 %6, %12 offset:14336\n\t"
            "ds_read_b128 %7, %13 offset:14336\n\t"
            "ds_read_b32 %8, %14 offset:256\n\t"
            "ds_read_b32 %9, %14 offset:320\n\t"
            "ds_read_b32 %10, %14 offset:384\n\t"
            "ds_read_b32 %11, %14 offset:448\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(al[MT > 4 ? 4 : 0]), "=&v"(ah[MT > 4 ? 4 : 0]), "=&v"(al[MT > 5 ? 5 : 0]),
              "=&v"(ah[MT > 5 ? 5 : 0]), "=&v"(al[MT > 6 ? 6 : 0]), "=&v"(ah[MT > 6 ? 6 : 0]),
              "=&v"(al[MT > 7 ? 7 : 0]), "=&v"(ah[MT > 7 ? 7 : 0]), "=&v"(sa[MT > 4 ? 4 : 0]),
              "=&v"(sa[MT > 5 ? 5 : 0]), "=&v"(sa[MT > 6 ? 6 : 0]), "=&v"(sa[MT > 7 ? 7 : 0])
            : "v"(a0), "v"(a1), "v"(sp)
            : "memory");
      }
    }
    v8i wf;
    wf[0] = wl[0]; wf[1] = wl[1]; wf[2] = wl[2]; wf[3] = wl[3];
    wf[4] = wh[0]; wf[5] = wh[1]; wf[6] = wh[2]; wf[7] = wh[3];
    // (schemes 1 and 2 copy no activation scales: their sa reads see stale bytes, unused)
    const float sw = SCH == 2 ? 0.0f : sws[kk];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      v8i bf;
      bf[0] = al[j][0]; bf[1] = al[j][1]; bf[2] = al[j][2]; bf[3] = al[j][3];
      bf[4] = ah[j][0]; bf[5] = ah[j][1]; bf[6] = ah[j][2]; bf[7] = ah[j][3];
      if constexpr (SCH == 0) acc[j] += mfma_e4m3_16x16x128(wf, bf) * (sa[j] * sw);
      else if constexpr (SCH == 1) acc[j] += mfma_f8_16x16x128<CODE>(wf, bf, v4f{0.0f, 0.0f, 0.0f, 0.0f}) * sw;
      else acc[j] = mfma_f8_16x16x128<CODE>(wf, bf, acc[j]);
    }
  };

  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(min(i, nk - 1), stage(i));
    for (int kk = 0; kk < nk; kk += D) {
#pragma unroll
      for (int i = 0; i < D; ++i)
        if (kk + i < nk) step(kk + i, stage(i), stage((i + D - 1) % D));
    }
  }
  // the clamped copies past the slice must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());

  const int64_t n = n0 + 16 * wave + 4 * g;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int64_t m = 16 * j + r;
    if (m < M) {
      if (S == 1) {
        if constexpr (SCH != 0) {
          // scales that do not vary along K: the token's (or the tensor's), then the channels'
          // (sliced calls apply them in the reduction)
          acc[j] = acc[j] * gload<float>(p.s_a + (p.a_kind == 2 ? 0 : m));
          if constexpr (SCH == 2) acc[j] = acc[j] * gload<v4f>(reinterpret_cast<const float*>(p.s_w) + n);
        }
        store4<OUT>(p.y, p.ldy, m, n, acc[j]);
      } else {
        gstore<v4f>(ws + ((int64_t)split * M + m) * N + n, acc[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// M <= 16: one workgroup per 16 weight rows and the whole K, its WK waves splitting the K-blocks
// (contiguous slices) and adding their 16x16 partial tiles through LDS in wave order.  No
// workspace, one launch.  Each K-block's 16 x 128-byte weight tile is loaded as whole lines (lane
// l: row l/8 and row l/8 + 8, bytes 16 (l%8) .. +15; each load instruction covers 8 full lines)
// two blocks per register chunk, two chunks in flight, and reordered into the MFMA operand
// layout through a per-wave LDS tile (two 16-byte writes and two reads per lane per block).
// Loaded straight in the operand layout (16 rows x 32 bytes per lane group) every instruction
// touched 16 half-used lines and cost ~4x the address-unit time per byte; measured (graph loop)
// 6144x4096 at M = 8 9.1 -> 7.6 us, 24576x1536 10.0 -> 8.5 us, and the 28672x4096 weight, which
// used to take the LDS-ring kernel, 25.0 -> 21.9 us at M = 1.  The activation fragments come
// straight from L2 (the whole activation is at most 16 rows).
// ---------------------------------------------------------------------------------------------
constexpr int CHS = 2;  // K-blocks per register chunk in the small-M kernel (4: no faster)

// MODE (MoE with at most 64 rows per expert, grid.y = expert e): 1 = the expert's rows are
// offsets[e] .. offsets[e+1]-1 of the contiguous grouped layout; 2 = rows e*slot .. e*slot +
// counts[e] - 1 of the masked batched layout.  The workgroup walks its expert's rows in passes of
// up to 16 * MT_MAX rows (MT_MAX = 2: two 16-row tiles share each weight fragment, one K-block
// per register chunk), each pass streaming the weight tile again (a pass after the first mostly
// from the last-level cache), and a workgroup whose expert has no rows exits after its 4-byte
// count load, so only routed experts' weights are read.  Every row's sums are those of a 16-row
// pass (same K split, block order and reduction order).  SCH and CODE as for the ring kernel
// (MoE layouts: scheme 0 only).
// (at least 3 waves per SIMD: with both pass variants of the MoE walk, the 16-row form would
// otherwise take 172 VGPRs and run 2 waves per SIMD, 13-25% slower on MoE down)
template <int WK, int SWF, int OUT, int MODE = 0, int SCH = 0, int CODE = 0, int MT_MAX = 1>
__global__ __launch_bounds__(64 * WK, 3) void gemm_decode_small_kernel(GemmArgs p) {
  static_assert(SCH != 0 || CODE == 0, "the 1x128-group scheme runs on E4M3 operands");
  static_assert(MODE == 0 || SCH == 0, "MoE layouts use the 1x128-group scheme");
  static_assert(MT_MAX == 1 || MT_MAX == 2, "16-row tiles per pass: 1 or 2");
  static_assert(MODE != 0 || MT_MAX == 1, "at most 16 rows without an expert layout");
  __shared__ v4f red[WK > 1 ? WK - 1 : 1][MT_MAX][64];
  __shared__ __attribute__((aligned(1024))) uint8_t tile[WK][CHS][16 * 128];  // per wave, per block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this workgroup's rows: row_base .. r_end - 1 (MoE: the expert's rows, in passes of 16)
  int64_t row_base = 0, r_end = p.M, ex = 0;
  if constexpr (MODE != 0) {
    ex = blockIdx.y;
    int64_t r0, r1;
    if constexpr (MODE == 1) {  // (offsets are a precondition; clamped to 0..total rows)
      r0 = min(max((int64_t)gload<int>(p.offsets + ex), (int64_t)0), p.M);
      r1 = min(max((int64_t)gload<int>(p.offsets + ex + 1), r0), p.M);
    } else {
      r0 = ex * p.slot;
      r1 = r0 + min(max((int64_t)gload<int>(p.offsets + ex), (int64_t)0), p.slot);
    }
    row_base = __builtin_amdgcn_readfirstlane((int)r0);
    r_end = __builtin_amdgcn_readfirstlane((int)r1);
    if (r_end <= row_base) return;
  }
  const int64_t K = p.K;
  const int KB = (int)(K / 128);
  const int per = (KB + WK - 1) / WK;
  const int kb0 = min(KB, wave * per);
  const int nk = min(KB, kb0 + per) - kb0;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nb = n0 / 128;
  const int g = lane >> 4, r = lane & 15;
  const uint8_t* wline = p.w_q + (ex * p.N + n0 + (lane >> 3)) * K + (int64_t)kb0 * 128 + 16 * (lane & 7);
  const int64_t swbase = (ex * (p.N / 128) + nb) * KB + kb0;
  // LDS tile offsets: whole-line writes (rows l/8 and l/8 + 8, chunk l%8), operand-layout reads
  // (row l%16, logical chunks 2g and 2g+1), both through the conflict-free swizzle
  const int wo0 = swz(lane >> 3, lane & 7), wo1 = swz((lane >> 3) + 8, lane & 7);
  const int ro0 = swz(r, 2 * g), ro1 = swz(r, 2 * g + 1);

  // One pass over the rows row_base .. row_base + M - 1 (M <= 16 MT) as MT tiles of 16 rows;
  // LAST: the workgroup's last read of its weight rows.
  auto pass = [&](auto mt_c, auto last_c, const int64_t row_base, const int64_t M) {
    constexpr int MT = decltype(mt_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    constexpr int CH = MT == 1 ? CHS : 1;  // K-blocks per register chunk
    const uint8_t* arow[MT];
    const float* sarow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = row_base + (16 * t + r < M ? 16 * t + r : M - 1);  // rows past M repeat row M-1
      arow[t] = p.a_q + m * p.lda + (int64_t)kb0 * 128 + 32 * g;
      sarow[t] = p.s_a + (int64_t)kb0 * p.ld_sa + m;
    }
    int4 wv[2][CH][2], av[2][CH][MT][2];
    float sav[2][CH][MT], swv[2][CH];
    auto load_chunk = [&](int c, int buf) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (c + u < nk) {
          const int64_t off = (int64_t)(c + u) * 128;
          if constexpr (LAST) {
            wv[buf][u][0] = gload_i4_last(wline + off);
            wv[buf][u][1] = gload_i4_last(wline + 8 * K + off);
          } else {
            wv[buf][u][0] = gload_i4(wline + off);
            wv[buf][u][1] = gload_i4(wline + 8 * K + off);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            av[buf][u][t][0] = gload_i4(arow[t] + off);
            av[buf][u][t][1] = gload_i4(arow[t] + off + 16);
            if constexpr (SCH == 0) sav[buf][u][t] = gload<float>(sarow[t] + (int64_t)(c + u) * p.ld_sa);
          }
          if constexpr (SCH != 2) swv[buf][u] = load_sw<SWF>(p.s_w, swbase + c + u);
        }
      }
    };
    v4f acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute_chunk = [&](int c, int buf) {
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (c + u < nk) {
          // (one wave's LDS operations complete in order: the reads see the writes, and the next
          // chunk's writes to this tile follow these reads)
          uint8_t* tl = &tile[wave][u][0];
          *reinterpret_cast<int4*>(tl + wo0) = wv[buf][u][0];
          *reinterpret_cast<int4*>(tl + wo1) = wv[buf][u][1];
          const int4 lo = *reinterpret_cast<const int4*>(tl + ro0);
          const int4 hi = *reinterpret_cast<const int4*>(tl + ro1);
          v8i af;
          af[0] = lo.x; af[1] = lo.y; af[2] = lo.z; af[3] = lo.w;
          af[4] = hi.x; af[5] = hi.y; af[6] = hi.z; af[7] = hi.w;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            v8i bf;
            bf[0] = av[buf][u][t][0].x; bf[1] = av[buf][u][t][0].y; bf[2] = av[buf][u][t][0].z; bf[3] = av[buf][u][t][0].w;
            bf[4] = av[buf][u][t][1].x; bf[5] = av[buf][u][t][1].y; bf[6] = av[buf][u][t][1].z; bf[7] = av[buf][u][t][1].w;
            if constexpr (SCH == 0) acc[t] += mfma_e4m3_16x16x128(af, bf) * (sav[buf][u][t] * swv[buf][u]);
            else if constexpr (SCH == 1) acc[t] += mfma_f8_16x16x128<CODE>(af, bf, v4f{0.0f, 0.0f, 0.0f, 0.0f}) * swv[buf][u];
            else acc[t] = mfma_f8_16x16x128<CODE>(af, bf, acc[t]);
          }
        }
      }
    };
    load_chunk(0, 0);
    for (int c = 0; c < nk; c += 2 * CH) {
      if (c + CH < nk) load_chunk(c + CH, 1);
      compute_chunk(c, 0);
      if (c + CH < nk) {
        if (c + 2 * CH < nk) load_chunk(c + 2 * CH, 0);
        compute_chunk(c + CH, 1);
      }
    }
    auto finish = [&](int t) {
      const int64_t ml = 16 * t + r;
      if (ml < M) {
        if constexpr (SCH != 0) {
          // scales that do not vary along K: the token's (or the tensor's), then the channels'
          acc[t] = acc[t] * gload<float>(p.s_a + (p.a_kind == 2 ? 0 : row_base + ml));
          if constexpr (SCH == 2) acc[t] = acc[t] * gload<v4f>(reinterpret_cast<const float*>(p.s_w) + n0 + 4 * g);
        }
        store4<OUT>(p.y, p.ldy, row_base + ml, n0 + 4 * g, acc[t]);
      }
    };
    if constexpr (WK > 1) {
      if (wave > 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave - 1][t][lane] = acc[t];
      }
      __syncthreads();
      if constexpr (MODE == 0) {
        if (wave > 0) return;
      }
      if (wave == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
#pragma unroll
          for (int w = 0; w < WK - 1; ++w) acc[t] += red[w][t][lane];
          finish(t);
        }
      }
      if constexpr (MODE != 0) __syncthreads();  // the next pass rewrites red
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t) finish(t);
    }
  };
  // The weight loads of the last pass carry the non-temporal hint; earlier passes leave the rows in
  // the cache for the next (measured: one pass +4-11% with the hint, a hinted load of rows that
  // are read again up to 12% slower).
  using one = std::integral_constant<int, 1>;
  using yes = std::true_type;
  using no = std::false_type;
  if constexpr (MODE == 0) {
    pass(one{}, yes{}, 0, p.M);
  } else {
    for (int64_t rb = row_base; rb < r_end;) {
      const int64_t left = r_end - rb;
      if (MT_MAX == 2 && left > 16) {
        using two = std::integral_constant<int, MT_MAX>;
        if (left <= 32) pass(two{}, yes{}, rb, left);
        else pass(two{}, no{}, rb, 32);
        rb += 32;
      } else {
        if (left <= 16) pass(one{}, yes{}, rb, left);
        else pass(one{}, no{}, rb, 16);
        rb += 16;
      }
    }
  }
}

}  // namespace
}  // namespace fgb
