// gemm_decode.hip — path selection and launches of the decode (M <= 128) block-scaled FP8 GEMM
// kernels of gemm_decode_kernels.hpp, and the scratch the library owns for callers that cannot
// allocate.
#include <mutex>

#include "gemm_decode_kernels.hpp"

namespace fgb {

namespace {

int small_waves(int64_t N, int64_t K) { return decode_small_waves(N, K); }

}  // namespace

// Waves splitting K per 16-row tile in the M <= 16 kernels: 8 for at most 256 tiles (one per CU),
// else 4 (and at most one per K-block).  Measured over the decode shapes at M = 1 and 8 (graph
// loop) against the earlier rule of about 4k waves in all (1 wave per tile for 1536 and more
// tiles): 24576x1536 at M = 1 9.4 -> 8.2 us, 28672x4096 25.0 -> 24.3 us; 4 beats 8 from 384
// tiles on (6144x4096: 7.6 vs 8.1 us) and 8 beats 4 at 256 tiles (4096x4096: 5.7 vs 5.9 us).
int decode_small_waves(int64_t N, int64_t K) {
  const int64_t tiles = N / 16;
  int wk = tiles <= 256 ? 8 : 4;
  while (wk > 1 && wk > K / 128) wk /= 2;
  return wk;
}

// M <= 16: weights from this size on with long rows (K >= 8192: long slices per wave, where the
// ring reaches its steady state) take the LDS-ring kernel, the others the register kernel.
// Measured (graph loop): 4096x14336 at M = 16 14.7 vs 15.4 us, 7168x18432 31.5 vs 33.9 us (ring
// ahead, equal at M <= 4); 28672x4096 at M = 1 25.0 vs 21.9 us (register kernel ahead).
constexpr int64_t kRingMinWeightBytes = 48ll << 20;
bool decode_ring(int64_t N, int64_t K) { return N * K >= kRingMinWeightBytes && K >= 8192; }

// 16 < M <= 64 with weights of at most 16 MiB (the 4096 x 4096 projection): the per-wave ring
// kernel (16 weight rows and the whole K per workgroup, 4 waves, 32 or 64 activation rows), one
// launch.  Measured against the shared-ring kernel below, whose K slicing needs a second launch
// at these sizes: 4096 x 4096 at M = 32 7.1 vs 10.0 us, M = 64 8.9 vs 11.5 us.  For larger
// weights the per-wave copies of all activation rows cost more than the second launch.
bool ring_mid_rows(int64_t N, int64_t K) { return N * K <= (16ll << 20); }

// K-blocks per workgroup of the 16 < M <= 128 kernel.  One slice when the weight blocks alone give
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

// Waves (16 weight rows each) per workgroup of the 16 < M <= 128 kernel.  With at most 32
// activation rows and 32-63 K-blocks, workgroups of 2 or 4 waves cover the weight rows without K
// slices (one launch), 2 when that gives at most 256 workgroups, else 4 up to 512; otherwise 8
// (one 128-row block).  Measured (graph loop, interleaved A/B, at M = 17/24/32): 6144x4096 with 2
// waves 10.0-10.1 vs 10.2/10.5/11.0 us (8 waves, 4 K slices + reduction), 28672x4096 with 4
// waves 25.5/25.9/26.5 vs 27.0/27.1/27.3 us (8 waves, one slice); at 64 rows (4 waves 30.3 vs
// 28.5), 12 K-blocks (24576x1536) or 112-144 (4096x14336, 7168x18432) 8 waves stay ahead.
int mid_waves(int64_t M, int64_t N, int64_t K) {
  if (M > 32 || K < 32 * 128 || K >= 64 * 128) return 8;
  if (N / 32 <= 256) return 2;
  if (N / 64 <= 512) return 4;
  return 8;
}

int decode_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || (M <= 64 && ring_mid_rows(N, K))) return 1;  // these kernels need no workspace
  if (mid_waves(M, N, K) < 8) return 1;
  const int KB = (int)(K / 128);
  const int kpw = mid_kpw(N, K);
  return (KB + kpw - 1) / kpw;
}

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = decode_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_decode(const GemmArgs& a, void* workspace, hipStream_t stream) {
  if (a.M <= 16 && decode_ring(a.N, a.K)) {
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
  if (a.M > 16 && a.M <= 64 && ring_mid_rows(a.N, a.K)) {
    const dim3 grid((unsigned)(a.N / 16));
#define FGB_RING_MID(SWF, OUT)                                                                                   \
  do {                                                                                                           \
    if (a.M <= 32) hipLaunchKernelGGL((gemm_decode_ring_kernel<4, 32, 3, SWF, OUT>), grid, dim3(256), 0, stream, a); \
    else hipLaunchKernelGGL((gemm_decode_ring_kernel<4, 64, 2, SWF, OUT>), grid, dim3(256), 0, stream, a);           \
  } while (0)
    if (a.s_w_fmt == 0) {
      if (a.y_dtype == 0) FGB_RING_MID(0, 0); else FGB_RING_MID(0, 1);
    } else {
      if (a.y_dtype == 0) FGB_RING_MID(1, 0); else FGB_RING_MID(1, 1);
    }
#undef FGB_RING_MID
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
    const int S = decode_splits(a.M, a.N, a.K);
    const int nw = mid_waves(a.M, a.N, a.K);
    const int kpw = S == 1 ? (int)(a.K / 128) : mid_kpw(a.N, a.K);
    const dim3 grid((unsigned)((a.N / (16 * nw)) * S)), block(64 * nw);
    float* ws = reinterpret_cast<float*>(workspace);
#define FGB_MID(NW_, MT_, D_, SWF, OUT) \
  hipLaunchKernelGGL((gemm_decode_mid_kernel<NW_, MT_, D_, SWF, OUT>), grid, block, 0, stream, a, kpw, S, ws)
#define FGB_MID_MT(SWF, OUT)                                    \
  do {                                                          \
    if (a.M > 64) FGB_MID(8, 8, kMidStages, SWF, OUT);          \
    else if (a.M > 32) FGB_MID(8, 4, kMidStages, SWF, OUT);     \
    else if (nw == 2) FGB_MID(2, 2, 6, SWF, OUT);               \
    else if (nw == 4) FGB_MID(4, 2, 4, SWF, OUT);               \
    else FGB_MID(8, 2, kMidStages, SWF, OUT);                   \
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
      hipLaunchKernelGGL(splitk_reduce_kernel<0>, rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy,
                         nullptr, 0, nullptr);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<1>, rgrid, dim3(256), 0, stream, ws, S, a.M, a.N, a.y, a.ldy,
                         nullptr, 0, nullptr);
    return hipGetLastError();
  }
}

// ---------------------------------------------------------------------------------------------
// MoE with at most 64 rows per expert (decode-shaped routing): the M <= 16 register kernel with
// grid.y = expert, 4 waves splitting K, one workgroup per (16 weight rows, expert) walking the
// expert's rows in passes of 16; mode 1 reads the contiguous grouped layout's offsets, mode 2 the
// masked batched layout's counts (slot = rows per expert slot).
//
// Measured (32 experts, graph loop, gate+up 4096x7168 / down 7168x2048): against the per-wave LDS
// ring kernel with 8 or 16 staged rows (the same K split, so the same bits) top-8 routing of 1
// token 41.9 -> 40.9 / 28.8 -> 22.5 us, of 8 tokens 136.5 -> 130.7 / 96.8 -> 66.8 us, 64-row
// batched slots for 64 tokens 236 -> 230 / 159 -> 119 us: down's 16 K-blocks give each wave 4,
// too few for a ring to fill.  Passes inside the workgroup rather than one workgroup per chunk
// of rows: the grid then holds no workgroups without rows, which hold a CU slot for the latency
// of their count load (ring kernel: 143 -> 136 and 109 -> 96 us at 8 tokens).
// ---------------------------------------------------------------------------------------------
namespace {

template <int MODE, int MTM>
void launch_moe(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N / 16), (unsigned)a.E), block(256);
  if (a.s_w_fmt == 0) {
    if (a.y_dtype == 0) hipLaunchKernelGGL((gemm_decode_small_kernel<4, 0, 0, MODE, 0, 0, MTM>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gemm_decode_small_kernel<4, 0, 1, MODE, 0, 0, MTM>), grid, block, 0, stream, a);
  } else {
    if (a.y_dtype == 0) hipLaunchKernelGGL((gemm_decode_small_kernel<4, 1, 0, MODE, 0, 0, MTM>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gemm_decode_small_kernel<4, 1, 1, MODE, 0, 0, MTM>), grid, block, 0, stream, a);
  }
}

}  // namespace

// Rows per weight pass: up to 32 (two 16-row tiles per weight fragment) when an expert can have
// more than 16 rows and K has at least 32 blocks, else 16.  Measured (32 experts, graph loop,
// interleaved A/B, bitwise equal outputs): 4096x7168 with 64-row batched slots for 64 / 32
// tokens 230 -> 215 / 176 -> 173 us, 8 / 16 tokens within 1%; on 7168x2048 (4 K-blocks per
// wave) two-tile passes were 7-10% slower below 64 tokens, passes of 64 rows (212 VGPRs: half
// the waves per SIMD) slower everywhere but 4096x7168 at 64 tokens.
namespace {
int moe_rows_per_pass(const GemmArgs& a, int mode) {
  const int64_t most = mode == 1 ? a.M : a.slot;  // most rows one expert can have
  return most > 16 && a.K >= 32 * 128 ? 32 : 16;
}
}  // namespace

hipError_t launch_gemm_moe_decode(const GemmArgs& a, int mode, hipStream_t stream) {
  const bool two = moe_rows_per_pass(a, mode) == 32;
  if (mode == 1) {
    if (two) launch_moe<1, 2>(a, stream);
    else launch_moe<1, 1>(a, stream);
  } else {
    if (two) launch_moe<2, 2>(a, stream);
    else launch_moe<2, 1>(a, stream);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, int S, int64_t M, int64_t N, void* y, int y_dtype, int64_t ldy,
                                hipStream_t stream) {
  const int64_t total = M * (N / 4);
  const dim3 rgrid((unsigned)((total + 255) / 256));
  if (y_dtype == 0)
    hipLaunchKernelGGL(splitk_reduce_kernel<0>, rgrid, dim3(256), 0, stream, ws, S, M, N, y, ldy, nullptr, 0, nullptr);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, rgrid, dim3(256), 0, stream, ws, S, M, N, y, ldy, nullptr, 0, nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Library-owned scratch for callers that cannot allocate (the no-allocation GEMM entry point).
// One array per GPU, in the code object's device memory for as long as the library is loaded.
// Host code never uses the array's name as an address: hipGetSymbolAddress gives each device's
// own copy, looked up once per device and kept.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace fgb
