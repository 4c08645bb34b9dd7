// gemm_prefill.hip — block-scaled FP8 W8A8 GEMM for M > 64, dense and grouped (MoE), gfx950.
//
// y[m, n] = sum_kb s_a[m, kb] * s_w[n/128, kb] * (A_q[m, kb-block] . W_q[n, kb-block])
// (Transformers "Fine-grained FP8", "DeepGEMM fast path"; grouped: the expert matmuls of the
// same section and of "UE8M0 scale format").
//
// Workgroup: 256 threads (4 waves) computing a BN x BM tile of y^T (BN output features x BM
// tokens).  Per K-block the W and A tiles (BN x 128 and BM x 128 bytes) are staged through LDS,
// double-buffered: the global loads for block kb+1 are in flight while block kb is multiplied.
// LDS rows are 128 bytes; 16-byte chunk c of row r lives at chunk c ^ (r & 7), so the 8 lanes
// of a ds_read_b128 phase hit 8 different bank groups.
//
// Each wave owns a (BN/2) x (BM/2) sub-tile = TN x TM MFMA tiles of 16x16.  For every K-block
// one MFMA per tile yields the exact-product float32 partial P, and acc += P * (s_a * s_w).
#include "gemm_common.hpp"
#include "internal.h"

namespace fgb {

namespace {

constexpr int THREADS = 256;
constexpr int KBYTES = 128;  // one K-block of E4M3 codes per row

template <int BN, int BM>
struct Tile {
  static constexpr int TN = BN / 2 / 16;  // MFMA tiles per wave along n
  static constexpr int TM = BM / 2 / 16;  // along m
  static constexpr int W_LOADS = BN * KBYTES / 16 / THREADS;  // 16 B chunks per thread
  static constexpr int A_LOADS = BM * KBYTES / 16 / THREADS;
  static constexpr int W_BYTES = BN * KBYTES;
  static constexpr int A_BYTES = BM * KBYTES;
  static constexpr int STAGE = W_BYTES + A_BYTES;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * KBYTES + ((chunk ^ (row & 7)) << 4); }

// Read one 16 x 128 fragment (lane row = lane%16, bytes 32g .. 32g+31 with g = lane/16).
__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int g = lane >> 4;
  const int4 lo = *reinterpret_cast<const int4*>(base + swz(r, 2 * g));
  const int4 hi = *reinterpret_cast<const int4*>(base + swz(r, 2 * g + 1));
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

struct RowRange {
  int64_t row0;     // first activation row of this tile
  int64_t row_end;  // one past the last valid row (expert end or M)
  int64_t expert;
};

template <int BN, int BM, int SWF, int OUT, bool GROUPED>
__global__ __launch_bounds__(THREADS, 2) void gemm_prefill_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  using T = Tile<BN, BM>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  const int nwg = tiles_m * tiles_n;
  const int pid = xcd_remap((int)blockIdx.x, nwg);
  // grouped ordering: bands of GROUP_M tile-rows share W tiles in L2
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * tiles_n;
  const int group_id = pid / in_group;
  const int first_m = group_id * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int pid_m = first_m + (pid % in_group) % gsize;
  const int pid_n = (pid % in_group) / gsize;

  const int64_t K = p.K, N = p.N;
  const int KB = (int)(K / KBYTES);
  const int NBLK = (int)(N / 128);

  RowRange rr;
  const uint8_t* wq = p.w_q;
  int64_t sw_base = 0;
  if constexpr (GROUPED) {
    // find the expert owning logical m-tile pid_m
    int cum = 0;
    int e = 0;
    int64_t r0 = 0, r1 = 0;
    bool found = false;
    for (; e < p.E; ++e) {
      r0 = p.offsets[e];
      r1 = p.offsets[e + 1];
      const int mt = (int)((r1 - r0 + BM - 1) / BM);
      if (pid_m < cum + mt) { found = true; break; }
      cum += mt;
    }
    if (!found) return;  // padding tile beyond the real tile count
    rr.row0 = r0 + (int64_t)(pid_m - cum) * BM;
    rr.row_end = r1;
    rr.expert = e;
    wq += (int64_t)e * N * K;
    sw_base = (int64_t)e * NBLK * KB;
  } else {
    rr.row0 = (int64_t)pid_m * BM;
    rr.row_end = p.M;
    rr.expert = 0;
  }
  const int64_t n0 = (int64_t)pid_n * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;

  // global -> register staging addresses
  const int ld_chunk = tid & 7;
  const int ld_row = tid >> 3;  // + 32 * i
  const uint8_t* wsrc[T::W_LOADS];
  const uint8_t* asrc[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::W_LOADS; ++i)
    wsrc[i] = wq + (n0 + ld_row + 32 * i) * K + ld_chunk * 16;
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int64_t row = rr.row0 + ld_row + 32 * i;
    row = row < rr.row_end ? row : rr.row_end - 1;
    asrc[i] = p.a_q + row * p.lda + ld_chunk * 16;
  }
  // per-lane activation scale rows (one token per lane per m-tile)
  int64_t sa_row[T::TM];
#pragma unroll
  for (int j = 0; j < T::TM; ++j) {
    int64_t row = rr.row0 + wm * (BM / 2) + j * 16 + (lane & 15);
    sa_row[j] = row < rr.row_end ? row : rr.row_end - 1;
  }
  const int64_t nb = (n0 + wn * (BN / 2)) / 128;  // weight block row of this wave (uniform)

  int4 wreg[T::W_LOADS], areg[T::A_LOADS];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i) wreg[i] = *reinterpret_cast<const int4*>(wsrc[i] + (int64_t)kb * KBYTES);
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) areg[i] = *reinterpret_cast<const int4*>(asrc[i] + (int64_t)kb * KBYTES);
  };
  auto sstore = [&](int buf) {
    uint8_t* ws = smem + buf * T::STAGE;
    uint8_t* as = ws + T::W_BYTES;
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i) *reinterpret_cast<int4*>(ws + swz(ld_row + 32 * i, ld_chunk)) = wreg[i];
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) *reinterpret_cast<int4*>(as + swz(ld_row + 32 * i, ld_chunk)) = areg[i];
  };

  v4f acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  float sa_cur[T::TM], sa_nxt[T::TM];
  float sw_cur, sw_nxt = 0.0f;
  gload(0);
#pragma unroll
  for (int j = 0; j < T::TM; ++j) sa_cur[j] = p.s_a[sa_row[j]];
  sw_cur = load_sw<SWF>(p.s_w, sw_base + nb * KB);
  sstore(0);
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < KB;
    if (more) {
      gload(kb + 1);
#pragma unroll
      for (int j = 0; j < T::TM; ++j) sa_nxt[j] = p.s_a[(int64_t)(kb + 1) * p.ld_sa + sa_row[j]];
      sw_nxt = load_sw<SWF>(p.s_w, sw_base + nb * KB + kb + 1);
    }
    const uint8_t* ws = smem + buf * T::STAGE;
    const uint8_t* as = ws + T::W_BYTES;
    v8i bf[T::TM];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) bf[j] = lds_frag(as, wm * (BM / 2) + j * 16, lane);
    float sc[T::TM];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) sc[j] = sa_cur[j] * sw_cur;
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      const v8i af = lds_frag(ws, wn * (BN / 2) + i * 16, lane);
#pragma unroll
      for (int j = 0; j < T::TM; ++j) {
        const v4f P = mfma_e4m3_16x16x128(af, bf[j]);
        acc[i][j] += P * sc[j];
      }
    }
    if (more) {
      sstore(buf ^ 1);
#pragma unroll
      for (int j = 0; j < T::TM; ++j) sa_cur[j] = sa_nxt[j];
      sw_cur = sw_nxt;
    }
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int j = 0; j < T::TM; ++j) {
    const int64_t m = rr.row0 + wm * (BM / 2) + j * 16 + (lane & 15);
    if (m < rr.row_end) {
#pragma unroll
      for (int i = 0; i < T::TN; ++i) {
        const int64_t n = n0 + wn * (BN / 2) + i * 16 + 4 * (lane >> 4);
        store4<OUT>(p.y, p.ldy, m, n, acc[i][j]);
      }
    }
  }
}

constexpr int BN_ = 128, BM_ = 128;

template <bool GROUPED>
hipError_t launch_impl(const GemmArgs& a, int tiles_m, hipStream_t stream) {
  const int tiles_n = (int)(a.N / BN_);
  const int nwg = tiles_m * tiles_n;
  dim3 grid(nwg), block(THREADS);
#define FGB_LAUNCH(SWF, OUT)                                                                   \
  hipLaunchKernelGGL((gemm_prefill_kernel<BN_, BM_, SWF, OUT, GROUPED>), grid, block, 0, stream, a, \
                     tiles_m, tiles_n)
  if (a.s_w_fmt == 0 && a.y_dtype == 0) FGB_LAUNCH(0, 0);
  else if (a.s_w_fmt == 0) FGB_LAUNCH(0, 1);
  else if (a.y_dtype == 0) FGB_LAUNCH(1, 0);
  else FGB_LAUNCH(1, 1);
#undef FGB_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, hipStream_t stream) {
  const int tiles_m = (int)((a.M + BM_ - 1) / BM_);
  return launch_impl<false>(a, tiles_m, stream);
}

hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t stream) {
  // upper bound on the per-expert tile count: sum_e ceil(M_e/BM) <= ceil(total_M/BM) + E
  const int tiles_m = (int)((a.M + BM_ - 1) / BM_) + a.E;
  return launch_impl<true>(a, tiles_m, stream);
}

}  // namespace fgb
