// gemm_decode.hip — block-scaled FP8 GEMM for small M (decode, M <= 64), gfx950.
//
// Same result as the prefill path (Transformers "Fine-grained FP8", "DeepGEMM fast path"), but
// for few tokens the weight stream dominates (bytes per weight: 1 for FP8, per the Baseten
// NVFP4 summary, "Less memory, more compute"), so the kernels are organised to keep HBM busy:
//   * M <= 16: one workgroup per 16 weight rows and the whole K, its waves splitting the
//     K-blocks; weights >= 48 MiB stream through per-wave LDS rings with whole-line direct
//     copies, smaller ones load the MFMA operand layout straight into registers.  One launch.
//   * 16 < M <= 64: a workgroup of 8 waves per 128-row weight block over a K slice, weights,
//     activations and their scales streamed through a 4-stage LDS ring shared by the waves; K is
//     sliced only to occupy the CUs, and sliced shapes add their float32 partials [S][M][N] in a
//     second, ordered launch.  (A reduction inside the same launch would need device-scope
//     release fences, which on this multi-XCD part write back the L2 and cost more than the
//     second launch.)
#include "gemm_common.hpp"
#include "internal.h"

namespace fgb {

namespace {

// 16-byte chunk c of LDS row r sits at c ^ ((r & 7) ^ (r>>3 & 1)): conflict-free 16-row fragment
// reads on gfx950's 64-bank LDS.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

// Sum of the S partial slices in slice order; all loads of a group of 8 slices are issued
// before they are added.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int S, int64_t M,
                                                            int64_t N, void* y, int64_t ldy) {
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
  store4<OUT>(y, ldy, m, n, s);
}

#define GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int V>
constexpr int vmcnt_only() { return (V & 0xF) | ((V >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// gfx950 LDS: 16-byte chunk c of 128-byte row r at c ^ ((r & 7) ^ (r>>3 & 1))
__device__ __forceinline__ int swz_g(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// ---------------------------------------------------------------------------------------------
// M <= 16, large weights: same work split as the kernel below, but each wave streams its 16
// weight rows (and the <= MR activation rows of its K-slice, and their scales) through a private
// LDS ring of D stages with direct copies.  A copy instruction reads 8 whole 128-byte lines,
// where loading the MFMA operand layout straight into registers touches 16 half-used lines per
// instruction, which costs about four times as much address-unit time per byte on gfx950 and
// limits the weight stream below the HBM rate.  No barrier is needed until the partial tiles are
// added.  For small weights the extra LDS round trip costs more than it saves.
template <int WK, int MR, int D, int SWF, int OUT>
__global__ __launch_bounds__(64 * WK) void gemm_decode_ring_kernel(GemmArgs p) {
  constexpr int WST = 16 * 128, AST = MR * 128, SST = 64 * 4;
  constexpr int STAGE = WST + AST + SST;
  constexpr int OPS = 2 + MR / 8 + 1;  // direct copies per stage
  __shared__ __attribute__((aligned(1024))) uint8_t ring[WK * D * STAGE];
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

  // copy sources: lane i of 8-row group q takes row 8q + i/8, logical chunk (i%8) ^ g(row)
  uint32_t woff[2], aoff[MR / 8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * q + (lane >> 3);
    woff[q] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
#pragma unroll
  for (int q = 0; q < MR / 8; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int64_t m = r < M ? r : M - 1;
    aoff[q] = (uint32_t)(m * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint32_t soff = (uint32_t)(((lane & 15) < M ? (lane & 15) : M - 1) * 4);
  const uint8_t* wbase = p.w_q + n0 * K;

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
      __builtin_amdgcn_global_load_lds(GPTR(wb + o), LPTR(st + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < MR / 8; ++q) {
      uint32_t o = aoff[q];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(GPTR(ab + o), LPTR(st + WST + q * 1024), 16, 0, 0);
    }
    uint32_t o = soff;
    asm volatile("" : "+v"(o));
    __builtin_amdgcn_global_load_lds(GPTR(sb + o), LPTR(st + WST + AST), 4, 0, 0);
  };

  // weight-block scales of this wave's slice, lane l holding block kb0 + l + 64 t (K <= 32768)
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

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(min(i, nk - 1));
    for (int kk = 0; kk < nk; ++kk) {
      // refill the stage consumed one block ago (clamped past the slice: never a pending stage)
      issue(min(kk + D - 1, nk - 1));
      __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * OPS>());
      // The LDS reads are written as one asm block that also waits for them: the compiler cannot
      // tell this wave's ring stages apart and would otherwise wait for every copy in flight.
      const uint32_t st = (uint32_t)(uintptr_t)LPTR(wring + (kk % D) * STAGE);
      const int r = lane & 15, g = lane >> 4;
      const uint32_t aw0 = st + swz(r, 2 * g), aw1 = st + swz(r, 2 * g + 1);
      const int ra = r & (MR - 1);
      const uint32_t aa0 = st + WST + swz(ra, 2 * g), aa1 = st + WST + swz(ra, 2 * g + 1);
      const uint32_t as = st + WST + AST + 4 * r;
      v4i w0, w1, a0, a1;
      float sa;
      asm volatile(
          "ds_read_b128 %0, %5\n\t"
          "ds_read_b128 %1, %6\n\t"
          "ds_read_b128 %2, %7\n\t"
          "ds_read_b128 %3, %8\n\t"
          "ds_read_b32 %4, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(w0), "=&v"(w1), "=&v"(a0), "=&v"(a1), "=&v"(sa)
          : "v"(aw0), "v"(aw1), "v"(aa0), "v"(aa1), "v"(as)
          : "memory");
      v8i wf, af;
      wf[0] = w0[0]; wf[1] = w0[1]; wf[2] = w0[2]; wf[3] = w0[3];
      wf[4] = w1[0]; wf[5] = w1[1]; wf[6] = w1[2]; wf[7] = w1[3];
      af[0] = a0[0]; af[1] = a0[1]; af[2] = a0[2]; af[3] = a0[3];
      af[4] = a1[0]; af[5] = a1[1]; af[6] = a1[2]; af[7] = a1[3];
      acc += mfma_e4m3_16x16x128(wf, af) * (sa * sw_at(kk));
    }
  }
  // the clamped copies past the slice must land before the workgroup's LDS is released
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
// 16 < M <= 64: a workgroup of 8 waves owns one 128-row weight block (16 rows per wave) over a
// slice of K-blocks.  The block's weight rows, the 16*MT activation rows (rows >= M repeat row
// M-1; their results are dropped) and the activation scales of each K-block stream through a
// ring of D LDS stages shared by the waves, with whole-line buffer-form direct copies issued
// D-1 blocks ahead and one barrier per block; the activation stream is read once per 128 weight
// rows.  Slices (S > 1) write float32 partials [S][M][N] for the ordered reduction launch.
// ---------------------------------------------------------------------------------------------
template <int MT, int D, int SWF, int OUT>
__global__ __launch_bounds__(512, 1) void gemm_decode_mid_kernel(GemmArgs p, int kpw, int S, float* ws) {
  constexpr int MROWS = 16 * MT;
  constexpr int WB = 128 * 128, AB = MROWS * 128, SB = 64 * 4;
  constexpr int STAGE = WB + AB + SB;
  constexpr int A_GRP = MROWS / 8;                 // 8-row copy groups of the activation rows
  constexpr int OPS = 2 + 1 + 1;                   // copies per wave per block: W, A, scales
  static_assert(D >= 3 && D <= 6, "three to six stages");
  static_assert(MT == 2 || MT == 4, "32 or 64 activation rows");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[D > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st4[D > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st5[D > 5 ? STAGE : 16];
  __shared__ float sws[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = p.K, N = p.N, M = p.M;
  const int KB = (int)(K / 128);
  const int nt = blockIdx.x / S, split = blockIdx.x - nt * S;
  const int kb0 = split * kpw;
  const int nk = min(KB, kb0 + kpw) - kb0;
  const int64_t n0 = (int64_t)nt * 128;

  // copy sources: lane i of 8-row group q takes row 8q + i/8, logical chunk (i%8) ^ g(row); the
  // activation groups past A_GRP repeat earlier ones (same bytes to the same place: no branch)
  uint32_t woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (wave + 8 * i) + (lane >> 3);
    woff[i] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const int aq = wave % A_GRP;
  uint32_t aoff;
  {
    const int r = 8 * aq + (lane >> 3);
    const int64_t m = r < M ? r : M - 1;
    aoff = (uint32_t)(m * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint32_t soff = (uint32_t)((lane < M ? lane : M - 1) * 4);

  auto issue = [&](int kk, uint8_t* st) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the builtins exist in the device pass only)
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_q + n0 * K), 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.s_a, 0, -1, 0x00020000);
    const int kb = kb0 + kk;
    const uint32_t koff = (uint32_t)kb * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, LPTR(st + (wave + 8 * i) * 1024), 16, woff[i], koff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, LPTR(st + WB + aq * 1024), 16, aoff, koff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rs, LPTR(st + WB + AB), 4, soff, (uint32_t)(kb * p.ld_sa * 4), 0, 0);
#endif
  };
  auto stage = [&](int i) -> uint8_t* {
    switch (i) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      case 3: return st3;
      case 4: return st4;
      default: return st5;
    }
  };

  for (int c = tid; c < nk; c += 512) sws[c] = load_sw<SWF>(p.s_w, (n0 / 128) * KB + kb0 + c);

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
    }
    v8i wf;
    wf[0] = wl[0]; wf[1] = wl[1]; wf[2] = wl[2]; wf[3] = wl[3];
    wf[4] = wh[0]; wf[5] = wh[1]; wf[6] = wh[2]; wf[7] = wh[3];
    const float sw = sws[kk];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      v8i bf;
      bf[0] = al[j][0]; bf[1] = al[j][1]; bf[2] = al[j][2]; bf[3] = al[j][3];
      bf[4] = ah[j][0]; bf[5] = ah[j][1]; bf[6] = ah[j][2]; bf[7] = ah[j][3];
      acc[j] += mfma_e4m3_16x16x128(wf, bf) * (sa[j] * sw);
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
      if (S == 1) store4<OUT>(p.y, p.ldy, m, n, acc[j]);
      else gstore<v4f>(ws + ((int64_t)split * M + m) * N + n, acc[j]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// M <= 16: one workgroup per 16 weight rows and the whole K, its WK waves splitting the K-blocks
// (contiguous slices) and adding their 16x16 partial tiles through LDS in wave order.  No
// workspace, one launch; the activation fragments come straight from L2 (the whole activation
// is at most 16 rows).
// ---------------------------------------------------------------------------------------------
constexpr int CHS = 2;  // K-blocks per register chunk in the small-M kernel (~100 VGPRs)

template <int WK, int SWF, int OUT>
__global__ __launch_bounds__(64 * WK) void gemm_decode_small_kernel(GemmArgs p) {
  __shared__ v4f red[WK > 1 ? WK - 1 : 1][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t K = p.K, M = p.M;
  const int KB = (int)(K / 128);
  const int per = (KB + WK - 1) / WK;
  const int kb0 = min(KB, wave * per);
  const int nk = min(KB, kb0 + per) - kb0;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nb = n0 / 128;
  const int g = lane >> 4;
  const int64_t m = (lane & 15) < M ? (lane & 15) : M - 1;  // rows past M repeat row M-1
  const uint8_t* wrow = p.w_q + (n0 + (lane & 15)) * K + (int64_t)kb0 * 128 + 32 * g;
  const uint8_t* arow = p.a_q + m * p.lda + (int64_t)kb0 * 128 + 32 * g;
  const float* sarow = p.s_a + (int64_t)kb0 * p.ld_sa + m;
  const int64_t swbase = nb * KB + kb0;

  int4 wv[2][CHS][2], av[2][CHS][2];
  float sav[2][CHS], swv[2][CHS];
  auto load_chunk = [&](int c, int buf) {
#pragma unroll
    for (int u = 0; u < CHS; ++u) {
      if (c + u < nk) {
        const int64_t off = (int64_t)(c + u) * 128;
        wv[buf][u][0] = gload_i4(wrow + off);
        wv[buf][u][1] = gload_i4(wrow + off + 16);
        av[buf][u][0] = gload_i4(arow + off);
        av[buf][u][1] = gload_i4(arow + off + 16);
        sav[buf][u] = gload<float>(sarow + (int64_t)(c + u) * p.ld_sa);
        swv[buf][u] = load_sw<SWF>(p.s_w, swbase + c + u);
      }
    }
  };
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute_chunk = [&](int c, int buf) {
#pragma unroll
    for (int u = 0; u < CHS; ++u) {
      if (c + u < nk) {
        v8i af, bf;
        af[0] = wv[buf][u][0].x; af[1] = wv[buf][u][0].y; af[2] = wv[buf][u][0].z; af[3] = wv[buf][u][0].w;
        af[4] = wv[buf][u][1].x; af[5] = wv[buf][u][1].y; af[6] = wv[buf][u][1].z; af[7] = wv[buf][u][1].w;
        bf[0] = av[buf][u][0].x; bf[1] = av[buf][u][0].y; bf[2] = av[buf][u][0].z; bf[3] = av[buf][u][0].w;
        bf[4] = av[buf][u][1].x; bf[5] = av[buf][u][1].y; bf[6] = av[buf][u][1].z; bf[7] = av[buf][u][1].w;
        const float sc = sav[buf][u] * swv[buf][u];
        acc += mfma_e4m3_16x16x128(af, bf) * sc;
      }
    }
  };
  load_chunk(0, 0);
  for (int c = 0; c < nk; c += 2 * CHS) {
    if (c + CHS < nk) load_chunk(c + CHS, 1);
    compute_chunk(c, 0);
    if (c + CHS < nk) {
      if (c + 2 * CHS < nk) load_chunk(c + 2 * CHS, 0);
      compute_chunk(c + CHS, 1);
    }
  }
  if constexpr (WK > 1) {
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) acc += red[w][lane];
  }
  if ((lane & 15) < M) store4<OUT>(p.y, p.ldy, lane & 15, n0 + 4 * g, acc);
}

// waves splitting K per 16-row tile for the small-M kernel: about 4k waves in total
int small_waves(int64_t N, int64_t K) {
  const int64_t tiles = N / 16;
  int wk = 1;
  while (wk < 8 && tiles * wk * 2 <= 4096 && wk * 2 <= K / 128) wk *= 2;
  return wk;
}

// weights from this size on take the LDS-ring kernel for M <= 16
constexpr int64_t kRingMinWeightBytes = 48ll << 20;

constexpr int MID_D = 4;  // LDS stages of the 16 < M <= 64 kernel (measured: 4 >= 5, 6)

// K-blocks per workgroup of the 16 < M <= 64 kernel.  One slice when the weight blocks alone give
// 160 or more workgroups; otherwise slices for about 224 workgroups (one per CU, most of the
// 256), each at least 8 blocks long (shorter slices spend their time filling the ring and their
// partials cost more than the extra CUs bring; measured on the decode shapes).
int mid_kpw(int64_t N, int64_t K) {
  const int KB = (int)(K / 128);
  const int64_t wgs = N / 128;
  int S = wgs >= 160 ? 1 : (int)((224 + wgs - 1) / wgs);
  const int smax = KB / 8 > 1 ? KB / 8 : 1;
  S = S > smax ? smax : S;
  return (KB + S - 1) / S;
}

}  // namespace

int decode_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 16) return 1;  // the small-M kernels need no workspace
  const int KB = (int)(K / 128);
  const int kpw = mid_kpw(N, K);
  return (KB + kpw - 1) / kpw;
}

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = decode_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_decode(const GemmArgs& a, void* workspace, hipStream_t stream) {
  if (a.M <= 16 && a.N * a.K >= kRingMinWeightBytes) {
    const int wk = small_waves(a.N, a.K);
    const dim3 grid((unsigned)(a.N / 16));
#define FGB_RING(WK, SWF, OUT)                                                                              \
  do {                                                                                                      \
    if (a.M <= 8) hipLaunchKernelGGL((gemm_decode_ring_kernel<WK, 8, 5, SWF, OUT>), grid, dim3(64 * WK), 0, stream, a); \
    else hipLaunchKernelGGL((gemm_decode_ring_kernel<WK, 16, 4, SWF, OUT>), grid, dim3(64 * WK), 0, stream, a);         \
  } while (0)
#define FGB_RING_WK(SWF, OUT)                  \
  do {                                         \
    if (wk == 1) FGB_RING(1, SWF, OUT);        \
    else if (wk == 2) FGB_RING(2, SWF, OUT);   \
    else if (wk == 4) FGB_RING(4, SWF, OUT);   \
    else FGB_RING(8, SWF, OUT);                \
  } while (0)
    if (a.s_w_fmt == 0) {
      if (a.y_dtype == 0) FGB_RING_WK(0, 0); else FGB_RING_WK(0, 1);
    } else {
      if (a.y_dtype == 0) FGB_RING_WK(1, 0); else FGB_RING_WK(1, 1);
    }
#undef FGB_RING_WK
#undef FGB_RING
    return hipGetLastError();
  }
  if (a.M <= 16) {
    const int wk = small_waves(a.N, a.K);
    const dim3 grid((unsigned)(a.N / 16));
#define FGB_SMALL(WK, SWF, OUT) \
  hipLaunchKernelGGL((gemm_decode_small_kernel<WK, SWF, OUT>), grid, dim3(64 * WK), 0, stream, a)
#define FGB_SMALL_WK(SWF, OUT)                  \
  do {                                          \
    if (wk == 1) FGB_SMALL(1, SWF, OUT);        \
    else if (wk == 2) FGB_SMALL(2, SWF, OUT);   \
    else if (wk == 4) FGB_SMALL(4, SWF, OUT);   \
    else FGB_SMALL(8, SWF, OUT);                \
  } while (0)
    if (a.s_w_fmt == 0) {
      if (a.y_dtype == 0) FGB_SMALL_WK(0, 0); else FGB_SMALL_WK(0, 1);
    } else {
      if (a.y_dtype == 0) FGB_SMALL_WK(1, 0); else FGB_SMALL_WK(1, 1);
    }
#undef FGB_SMALL_WK
#undef FGB_SMALL
    return hipGetLastError();
  }
  {
    const int kpw = mid_kpw(a.N, a.K);
    const int S = decode_splits(a.M, a.N, a.K);
    const dim3 grid((unsigned)((a.N / 128) * S)), block(512);
    float* ws = reinterpret_cast<float*>(workspace);
#define FGB_MID(MT_, SWF, OUT) \
  hipLaunchKernelGGL((gemm_decode_mid_kernel<MT_, MID_D, SWF, OUT>), grid, block, 0, stream, a, kpw, S, ws)
#define FGB_MID_MT(SWF, OUT)                     \
  do {                                           \
    if (a.M <= 32) FGB_MID(2, SWF, OUT);         \
    else FGB_MID(4, SWF, OUT);                   \
  } while (0)
    if (a.s_w_fmt == 0) {
      if (a.y_dtype == 0) FGB_MID_MT(0, 0); else FGB_MID_MT(0, 1);
    } else {
      if (a.y_dtype == 0) FGB_MID_MT(1, 0); else FGB_MID_MT(1, 1);
    }
#undef FGB_MID_MT
#undef FGB_MID
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || S == 1) return err;
    const int64_t total = a.M * (a.N / 4);
    const dim3 rgrid((unsigned)((total + 255) / 256));
    if (a.y_dtype == 0)
      hipLaunchKernelGGL(splitk_reduce_kernel<0>, rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<1>, rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy);
    return hipGetLastError();
  }
}

}  // namespace fgb
