// gemm_prefill.hip — launches of the prefill block-scaled FP8 GEMM kernels (dense: M > 128) of
// gemm_prefill_kernels.hpp, dense and grouped (MoE), for gfx950.
//
// A dense GEMM splits its output columns between 256 x 256 and 256 x 128 tiles so that the tiles
// fill whole waves of CUs; with more 256 x 256 tiles than CUs and a short K (grouped: up to 64
// K-blocks) one workgroup per CU walks the tiles (gemm_prefill_persistent_kernel) and overlaps
// the work between consecutive tiles.
#include "gemm_prefill_kernels.hpp"

namespace fgb {

namespace {


template <typename C, bool GROUPED>
hipError_t launch_cfg(const GemmArgs& a, int tiles_m, hipStream_t stream) {
  const int tiles_n = (int)(a.N / C::BN);
  // grouped: tiles_m is an upper bound; a multiple of 8 workgroups gives every XCD at least its
  // share of the real tiles
  const int nwg = GROUPED ? (tiles_m * tiles_n + 7) / 8 * 8 : tiles_m * tiles_n;
  dim3 grid(nwg), block(C::THREADS);
#define FGB_LAUNCH(SWF, OUT)                                                                  \
  hipLaunchKernelGGL((gemm_prefill_kernel<C, SWF, OUT, GROUPED>), grid, block, 0, stream, a, \
                     tiles_m, tiles_n)
  if (a.s_w_fmt == 0 && a.y_dtype == 0) FGB_LAUNCH(0, 0);
  else if (a.s_w_fmt == 0) FGB_LAUNCH(0, 1);
  else if (a.y_dtype == 0) FGB_LAUNCH(1, 0);
  else FGB_LAUNCH(1, 1);
#undef FGB_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    cached[dev] =
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cached[dev];
}

namespace {

template <typename C>
int64_t tiles_for(int64_t M, int64_t N) { return ((M + C::BM - 1) / C::BM) * (N / C::BN); }

// The persistent form for more 256 x 256 tiles than CUs when K has at most max_kb blocks.  Dense
// (16 blocks), where the work between tiles weighs most: measured +4-7% at 12-16 blocks; at 32
// (gate+up) +2% alone but 0.5% slower inside the Llama step, and 0.2-1.5% slower at 56-144
// blocks.  Grouped (64 blocks): a one-tile launch also looks up each tile's expert when it
// starts, which the persistent form does from registers; MoE gate+up (56 blocks) +2-4%.  An even
// K-block count (a multiple of 4 with UE8M0 scales, copied four to a dword), bf16 output and
// 32-bit output offsets.
bool use_persistent(const GemmArgs& a, int64_t max_kb) {
  const int64_t KB = a.K / KBYTES, tiles = tiles_for<Big>(a.M, a.N);
  return tiles > cu_count() && KB <= max_kb && KB % 2 == 0 && (a.s_w_fmt == 0 || KB % 4 == 0) && a.y_dtype == 0 &&
         a.M * a.ldy * 2 < (int64_t(1) << 32);
}


// Tile choice (N % 256 == 0; otherwise 128 x 128 tiles with 2 stages).  256 x 256 tiles (8 waves
// of 128 x 64, two stages) need K of at least 8 blocks; 256 x 128 tiles (three stages, 8 waves of
// 64 x 64: four token tiles per wave, so the pinned MFMA/FMA pipeline applies) take ~0.6 of a
// 256 x 256 tile's time (~20% slower per flop, measured at equal fill).  The output columns are
// split: the first n_big run as 256 x 256 tiles, the rest as 256 x 128 tiles, each part in its
// own launch, with n_big chosen to minimize the waves of tiles over the CUs (one tile per CU at
// a time), weighted 1 and 0.6.  Whole waves of big tiles plus one wave of half tiles can beat
// either tile alone: QKV at M = 4096 (384 big tiles) runs 256 big + 256 half tiles.
}  // namespace

int64_t big_columns(int64_t M, int64_t N, int64_t K) {
  if (K < 8 * KBYTES) return 0;
  const int64_t cus = cu_count(), nc = N / Big::BN;
  const int64_t tm_big = (M + Big::BM - 1) / Big::BM, tm_half = (M + Half::BM - 1) / Half::BM;
  auto waves = [&](int64_t tiles) { return (tiles + cus - 1) / cus; };
  int64_t best_c = nc;
  double best = 1e30;
  for (int64_t c = nc; c >= 0; --c) {  // on a tie the most big tiles
    const double t = (double)waves(tm_big * c) + 0.6 * (double)waves(tm_half * (nc - c));
    if (t < best - 1e-9) { best = t; best_c = c; }
  }
  return best_c * Big::BN;
}

// K slices for launches whose output tiles would leave most CUs idle (M a little above the decode
// sizes: e.g. 16 tiles of 256 x 128 for N = 4096 at M = 128, where one launch ran at 0.07 of HBM on
// 4096 x 14336).  Tiles are 256 x 128 (128 x 128 when N % 256 != 0); the number of slices S
// fills the CUs with one workgroup each (S * tiles <= CUs), keeps at least 4 K-blocks per slice
// and at most 16 slices, and keeps the float32 partials (S * M * N * 4 bytes) within the
// library's scratch size, so that the no-allocation entry point runs the same plan.  S = 1: the
// tiles are not sliced (at least half the CUs get a tile, or the partials would not fit).  With
// more than a quarter of the CUs busy unsliced, only slices of at least 16 K-blocks pay for the
// partials and the second launch (measured: 28672 x 4096 at M = 65-128, 2 slices of 16 blocks,
// 41-42 -> 34-38 us; 24576 x 1536, 2 slices of 6 blocks, 17.6-18.3 -> 19.5-23.9 us).
int prefill_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 64 || N <= 0 || K <= 0 || N % 128 || K % KBYTES) return 1;
  const bool half = N % Half::BN == 0;
  const int64_t bm = half ? Half::BM : Narrow::BM, bn = half ? Half::BN : Narrow::BN;
  const int64_t tiles = ((M + bm - 1) / bm) * (N / bn);
  const int64_t cus = cu_count();
  if (2 * tiles > cus) return 1;
  const int64_t KB = K / KBYTES;
  int64_t S = cus / tiles;
  if (S > KB / 4) S = KB / 4;
  if (S > 16) S = 16;
  const int64_t fit = (int64_t)(kScratchBytes / ((size_t)M * (size_t)N * sizeof(float)));
  if (S > fit) S = fit;
  if (S < 2) return 1;
  const int64_t kslice = (KB + S - 1) / S;
  if (4 * tiles > cus && kslice < 16) return 1;
  return (int)((KB + kslice - 1) / kslice);  // no empty slice
}

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = prefill_splits(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

namespace {

template <typename C>
hipError_t launch_sliced(const GemmArgs& a, int S, float* ws, hipStream_t stream) {
  const int KB = (int)(a.K / KBYTES);
  GemmArgs b = a;
  b.kslice = (KB + S - 1) / S;
  b.y = ws;
  b.y_dtype = 1;
  b.ldy = a.N;
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM), tiles_n = (int)(a.N / C::BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)S), block(C::THREADS);
  if (a.s_w_fmt == 0)
    hipLaunchKernelGGL((gemm_prefill_kernel<C, 0, 1, false, 0, 0, true>), grid, block, 0, stream, b, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<C, 1, 1, false, 0, 0, true>), grid, block, 0, stream, b, tiles_m, tiles_n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(ws, S, a.M, a.N, a.y, a.y_dtype, a.ldy, stream);
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, void* workspace, hipStream_t stream) {
  const int S = prefill_splits(a.M, a.N, a.K);
  if (S > 1) {
    float* ws = reinterpret_cast<float*>(workspace);
    return a.N % Half::BN == 0 ? launch_sliced<Half>(a, S, ws, stream) : launch_sliced<Narrow>(a, S, ws, stream);
  }
  if (a.N % Big::BN != 0 || a.N % Half::BN != 0)
    return launch_cfg<Narrow, false>(a, (int)((a.M + Narrow::BM - 1) / Narrow::BM), stream);
  const int64_t n_big = big_columns(a.M, a.N, a.K);
  if (n_big > 0) {
    GemmArgs b = a;
    b.N = n_big;
    const int tiles_m = (int)((b.M + Big::BM - 1) / Big::BM);
    if (use_persistent(b, 16)) {
      // one workgroup per CU (a multiple of 8, as the XCD mapping of tiles assumes)
      const dim3 grid(cu_count() / 8 * 8);
      if (b.s_w_fmt == 0)
        hipLaunchKernelGGL((gemm_prefill_persistent_kernel<Big, 0, false>), grid, dim3(Big::THREADS), 0, stream, b,
                           tiles_m, (int)(b.N / Big::BN));
      else
        hipLaunchKernelGGL((gemm_prefill_persistent_kernel<Big, 1, false>), grid, dim3(Big::THREADS), 0, stream, b,
                           tiles_m, (int)(b.N / Big::BN));
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      const hipError_t e = launch_cfg<Big, false>(b, tiles_m, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (n_big == a.N) return hipSuccess;
  // the remaining output columns: their weight rows, block-scale rows and output columns
  GemmArgs h = a;
  h.N = a.N - n_big;
  h.w_q = a.w_q + n_big * a.K;
  h.s_w = (const uint8_t*)a.s_w + (n_big / 128) * (a.K / KBYTES) * (a.s_w_fmt == 0 ? 4 : 1);
  h.y = (uint8_t*)a.y + n_big * (a.y_dtype == 0 ? 2 : 4);
  return launch_cfg<Half, false>(h, (int)((h.M + Half::BM - 1) / Half::BM), stream);
}

hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t stream) {
  // upper bound on the per-expert tile count: sum_e ceil(M_e/BM) <= ceil(total_M/BM) + E
  // (256 x 256 tiles from 8 K-blocks, as for the dense GEMM; MoE down, K = 2048: +15% over 256 x 128)
  if (a.N % Big::BN == 0 && a.K >= 8 * KBYTES) {
    const int tiles_m = (int)((a.M + Big::BM - 1) / Big::BM) + a.E;
    // the persistent form (the real tile count is known only on the device, the bound decides),
    // with at most 63 experts (one wave pass)
    if (a.E <= 63 && use_persistent(a, 64)) {
      const dim3 grid(cu_count() / 8 * 8);
      if (a.s_w_fmt == 0)
        hipLaunchKernelGGL((gemm_prefill_persistent_kernel<Big, 0, true>), grid, dim3(Big::THREADS), 0, stream, a,
                           tiles_m, (int)(a.N / Big::BN));
      else
        hipLaunchKernelGGL((gemm_prefill_persistent_kernel<Big, 1, true>), grid, dim3(Big::THREADS), 0, stream, a,
                           tiles_m, (int)(a.N / Big::BN));
      return hipGetLastError();
    }
    return launch_cfg<Big, true>(a, tiles_m, stream);
  }
  if (a.N % Half::BN == 0)
    return launch_cfg<Half, true>(a, (int)((a.M + Half::BM - 1) / Half::BM) + a.E, stream);
  return launch_cfg<Narrow, true>(a, (int)((a.M + Narrow::BM - 1) / Narrow::BM) + a.E, stream);
}

}  // namespace fgb
