// gemm_prefill_kernels.hpp — the prefill (M > 64) block-scaled FP8 GEMM kernels, dense and
// grouped; included by the translation units that instantiate and launch them.
//
// y[m, n] = sum_kb s_a[m, kb] * s_w[n/128, kb] * (A_q[m, kb-block] . W_q[n, kb-block])
// (Transformers "Fine-grained FP8", "DeepGEMM fast path"; grouped: the expert matmuls of the
// same section and of "UE8M0 scale format").
//
// Workgroup: 8 waves, 2 per SIMD (the 128 x 128 tile: 4 waves, 2 workgroups per CU), computing a
// BN x BM tile of y^T (BN output features x BM tokens).  Per K-block the W and A tiles (BN x 128
// and BM x 128 bytes) and the tile's activation scales are copied HBM/L2 -> LDS by direct-to-LDS
// loads (buffer_load_dwordx4 ... lds: no VGPR staging), STAGES deep (three for 256 x 128 tiles,
// two for 256 x 256 and 128 x 128): while block kb is multiplied out of one stage, the copies of
// the next blocks land in the others.
// Each stage is its own __shared__ array so the compiler can tell the in-flight copies from the
// LDS reads of the current stage and does not wait for them.
//
// LDS rows are 128 bytes; 16-byte chunk c of row r sits at chunk c ^ g(r), g(r) = (r & 7) ^ (r>>3 & 1).
// gfx950 serves a ds_read_b128 16 lanes per cycle from 64 banks, i.e. two 128-byte rows per bank
// line: the 16 rows of a fragment read at one logical chunk land on 16 distinct (row parity,
// chunk) pairs, so the read is conflict-free (and so is any 8-row subset).  g depends on r mod 16
// only, so every fragment (16 rows from a multiple of 16) uses the same per-lane address offsets.
// A direct load writes 64 lanes x 16 B contiguously (8 rows), so lane i of 8-row group q fetches
// the global chunk that belongs at its slot: row 8q + i/8, logical chunk (i%8) ^ g(8q + i/8).
//
// Each wave owns a (BN/WN) x (BM/WM) sub-tile = TN x TM MFMA tiles of 16x16.  For every K-block
// one MFMA per tile yields the exact-product float32 partial P, and acc += P * (s_a * s_w).
// bf16 output tiles are staged through LDS so that the (non-temporal) stores write whole lines.
//
// Launches (host code at the end): a dense GEMM splits its output columns between 256 x 256 and
// 256 x 128 tiles so that the tiles fill whole waves of CUs; with more 256 x 256 tiles than CUs
// and a short K (grouped: up to 64 K-blocks) one workgroup per CU walks the tiles
// (gemm_prefill_persistent_kernel) and overlaps the work between consecutive tiles.
#pragma once
#include "gemm_common.hpp"
#include "internal.h"

namespace fgb {

namespace {


constexpr int KBYTES = 128;  // one K-block of E4M3 codes per row
// The copies of the next block are issued spread over the first MFMAs of the current one, one
// every SPACING MFMAs, rather than in a burst after the barrier (+2-5% on the 256 x 256 tiles;
// later issue leaves the copies too little time).
constexpr int SPACING = 2;

#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int BN_, int BM_, int WN_, int WM_, int MINB_, int STAGES_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
  static constexpr int MINB = MINB_;      // workgroups per CU the register budget is sized for
  static constexpr int STAGES = STAGES_;  // LDS stages: copies run STAGES-1 K-blocks ahead
  static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
  static constexpr int WAVES = WN * WM;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TN = BN / WN / 16;  // MFMA tiles per wave along n
  static constexpr int TM = BM / WM / 16;  // along m
  static constexpr int W_BYTES = BN * KBYTES;
  static constexpr int A_BYTES = BM * KBYTES;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  static constexpr int W_LD = BN / 8 / WAVES;  // direct loads (8 rows each) per wave per stage
  static constexpr int A_LD = BM / 8 / WAVES;
  static constexpr int SA_LD = BM / 64;  // 64-token copies of the tile's activation scales
  static constexpr int NDMA = W_LD + A_LD;
  static_assert(SA_LD <= WAVES, "one activation-scale copy per wave at most");
  static_assert(W_LD >= 1 && A_LD >= 1, "every wave loads whole 8-row groups");
  static_assert((BN / WN) % 128 == 0 || 128 % (BN / WN) == 0, "a wave's rows stay in one weight block");
  static_assert(TM >= 4, "four or more token tiles per wave: the scale-FMAs run one W fragment behind");
};

// s_waitcnt immediate that waits until at most N vector-memory operations are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
constexpr int vmcnt_imm() { return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Workgroup barrier without a memory fence: LDS written by the direct copies is complete once
// each wave's own vmcnt wait returns, so only the execution barrier is needed.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier after LDS writes that other waves read next: LDS operations of different waves may be
// served out of order, so the wave's own writes are waited for first.
__device__ __forceinline__ void wg_barrier_after_lds_writes() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0), vmcnt and expcnt at their maxima
  wg_barrier();
}

__host__ __device__ constexpr int swz_g(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * KBYTES + ((chunk ^ swz_g(row)) << 4); }

// One 16 x 128 fragment: lane row = lane%16, logical bytes 32g .. 32g+31 with g = lane/16.
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

// Scaling schemes (SCH): 0 = 1x128 activation groups and 128x128 weight blocks, scaled per K-block;
// 1 = weight blocks scaled per K-block, one activation scale per token or per tensor applied in
// the epilogue; 2 = per-channel weight scales and per-token or per-tensor activation scales, both
// applied in the epilogue, so the MFMAs accumulate in place with no per-block factor.  CODE: the
// operands' format (0 E4M3, 1 E5M2; schemes 1 and 2 only).  SPLIT: K-sliced launch (dense, scheme
// 0, float32 output): workgroup (x, y) multiplies tile x over K-blocks y*kslice ..
// min((y+1)*kslice, K/128) - 1 and writes its float32 partial tile to slice y of y = [S][M][ldy].
template <typename C, int SWF, int OUT, bool GROUPED, int SCH = 0, int CODE = 0, bool SPLIT = false>
__global__ __launch_bounds__(C::THREADS, C::MINB) void gemm_prefill_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  static_assert(!SPLIT || (!GROUPED && SCH == 0 && OUT == 1), "K slices: dense block scheme, float32 partials");
  static_assert(SCH == 0 || SCH == 1 || SCH == 2, "scheme");
  static_assert(SCH != 0 || CODE == 0, "the 1x128-group scheme runs on E4M3 operands");
  // one __shared__ array per stage, so the compiler can tell in-flight copies from reads
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[C::STAGES > 2 ? C::STAGE : 16];
  // the tile's activation scales s_a[row0 .. row0+BM-1, kb], one array per stage like the tiles
  __shared__ __attribute__((aligned(16))) float sas0[C::BM];
  __shared__ __attribute__((aligned(16))) float sas1[C::BM];
  __shared__ __attribute__((aligned(16))) float sas2[C::STAGES > 2 ? C::BM : 4];

  const int64_t K = p.K, N = p.N;
  const int KBF = (int)(K / KBYTES);  // K-blocks of a row (the row pitch of s_w)
  // this workgroup's K-blocks: kb0 .. kb0 + KB - 1 (the whole row unless K is sliced)
  const int kb0 = SPLIT ? (int)blockIdx.y * p.kslice : 0;
  const int KB = SPLIT ? min(p.kslice, KBF - kb0) : KBF;
  const int NBLK = (int)(N / 128);

  // Grouped: tiles are numbered expert by expert, ceil(rows_e / BM) tile-rows each.  The grid is
  // an upper bound (host side the counts are unknown), so the real tiles are counted first and
  // split evenly over the XCDs; surplus workgroups exit.  (Numbering over the bound instead left
  // the padding on the last XCDs: for MoE down one XCD idle and 17.5 waves of tiles instead of
  // 15.75.)  63 experts per wave pass: lane l holds offsets[e0 + l], the tile-row counts are
  // prefix-summed across the wave; with at most 63 experts the one pass also finds the expert.
  const int lane0 = threadIdx.x & 63;
  auto expert_chunk = [&](int e0, int& off, int& nxt, int& mt, int& inc) {
    const int idx = e0 + lane0;
    // offsets are a precondition; clamped to 0..M, and an expert whose end lies before its start
    // gets no tiles, so that bad offsets cannot move a tile's rows outside 0..M-1.  Batched
    // layout: the slot's first row and its count (clamped to the slot)
    if (p.slot > 0) {
      off = idx < p.E ? idx * (int)p.slot : 0;
      nxt = idx < p.E ? off + min(max(gload<int>(p.offsets + idx), 0), (int)p.slot) : 0;
    } else {
      off = idx <= p.E ? min(max(gload<int>(p.offsets + idx), 0), (int)p.M) : 0;
      nxt = __shfl_down(off, 1);
    }
    mt = lane0 < 63 && idx < p.E && nxt > off ? (nxt - off + C::BM - 1) / C::BM : 0;
    inc = mt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(inc, d);
      if (lane0 >= d) inc += t;
    }
  };
  int c_off = 0, c_nxt = 0, c_mt = 0, c_inc = 0;  // the first chunk, kept for the lookup
  int real_tiles_m = tiles_m;
  if constexpr (GROUPED) {
    real_tiles_m = 0;
    for (int e0 = 0; e0 < p.E; e0 += 63) {
      int off, nxt, mt, inc;
      expert_chunk(e0, off, nxt, mt, inc);
      if (e0 == 0) { c_off = off; c_nxt = nxt; c_mt = mt; c_inc = inc; }
      real_tiles_m += __shfl(inc, 62);
    }
    real_tiles_m = min(real_tiles_m, tiles_m);  // (valid offsets never exceed the host's bound)
  }
  const int nwg = real_tiles_m * tiles_n;
  if (GROUPED && (int)blockIdx.x / 8 >= nwg / 8 + ((int)blockIdx.x % 8 < nwg % 8)) return;
  const int pid = xcd_remap((int)blockIdx.x, nwg);
  // grouped ordering: bands of GROUP_M tile-rows share W tiles in L2 (narrower bands for short K,
  // where a tile's operands are in L2 only briefly)
  const int GROUP_M = p.K <= 16 * KBYTES ? 4 : 8;
  const int in_group = GROUP_M * tiles_n;
  const int group_id = pid / in_group;
  const int first_m = group_id * GROUP_M;
  const int gsize = min(real_tiles_m - first_m, GROUP_M);
  const int pid_m = first_m + (pid % in_group) % gsize;
  const int pid_n = (pid % in_group) / gsize;

  int64_t row0, row_end;
  const uint8_t* wq = p.w_q;
  int64_t sw_base = 0;
  if constexpr (GROUPED) {
    // expert of tile-row pid_m: a ballot finds the first expert whose tile-rows reach past it
    int cum = 0, e = -1;
    int r0 = 0, r1 = 0;
    for (int e0 = 0; e0 < p.E; e0 += 63) {
      int off = c_off, nxt = c_nxt, mt = c_mt, inc = c_inc;
      if (e0 > 0) expert_chunk(e0, off, nxt, mt, inc);
      const unsigned long long hit = __ballot(mt > 0 && cum + inc > pid_m);
      if (hit) {
        const int first = __ffsll((long long)hit) - 1;
        e = e0 + first;
        r0 = __shfl(off, first);
        r1 = __shfl(nxt, first);
        cum += __shfl(inc - mt, first);
        break;
      }
      cum += __shfl(inc, 62);
    }
    if (e < 0) return;  // (cannot happen: the real tile count is the prefix sum searched here)
    row0 = (int64_t)r0 + (int64_t)(pid_m - cum) * C::BM;
    row_end = r1;
    wq += (int64_t)e * N * K;
    sw_base = (int64_t)e * NBLK * KBF;
  } else {
    row0 = (int64_t)pid_m * C::BM;
    row_end = p.M;
  }
  const int64_t n0 = (int64_t)pid_n * C::BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WN, wm = wave / C::WN;

  // direct-load sources: lane i of 8-row group q fetches row 8q + i/8, chunk (i%8) ^ g(row)
  const int lrow = lane >> 3;
  // 32-bit per-lane byte offsets from workgroup-uniform bases (the library checks that every
  // operand fits in 4 GiB): the base sits in the buffer descriptor, the offset in one VGPR
  uint32_t woff[C::W_LD], aoff[C::A_LD];
  const uint8_t* wbase = wq + n0 * K;
  const uint8_t* abase = p.a_q;
#pragma unroll
  for (int i = 0; i < C::W_LD; ++i) {
    const int q = wave + i * C::WAVES;
    const int r = 8 * q + lrow;
    woff[i] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int q = wave + i * C::WAVES;
    const int r = 8 * q + lrow;
    int64_t row = row0 + r;
    row = row < row_end ? row : row_end - 1;
    aoff[i] = (uint32_t)(row * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  // activation-scale copy: lane l of wave w fetches the scale of token row0 + 64 (w % SA_LD) + l
  // (clamped to the last row, like the tile rows).  Waves past SA_LD repeat a copy of an earlier
  // wave (same bytes to the same place) rather than skip it: a branch here would leave the
  // compiler unable to count the LDS reads that follow and make it wait for all of them.
  const int sa_grp = wave % C::SA_LD;
  uint32_t saoff;
  {
    int64_t row = row0 + 64 * sa_grp + lane;
    row = row < row_end ? row : row_end - 1;
    saoff = (uint32_t)(row * 4);
  }
  // The copies use the buffer form of the direct-to-LDS load (MUBUF).  The global form is a FLAT
  // instruction that touches both global memory and LDS, after which the compiler can no longer
  // count LDS reads and waits for all of them (lgkmcnt(0)) wherever it needs one; with buffer
  // loads it waits only for the reads the next instruction uses.  32-bit offsets; the range check
  // is off (num_records = 2^32 - 1): the library validated every operand's extent.
  // Copy d of block kb into stage st: 0 = the activation scales, then the W_LD weight and the
  // A_LD activation 8-row groups.
  // (schemes 1 and 2 have no per-block activation scales to copy: part 0 is skipped)
  constexpr int NPART = (SCH == 0 ? 1 : 0) + C::W_LD + C::A_LD;
  auto issue_part = [&](int kb, uint8_t* st, float* sas, int d) {
    if constexpr (SCH != 0) d += 1;
#if defined(__HIP_DEVICE_COMPILE__)  // (the builtins exist in the device pass only)
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.s_a, 0, -1, 0x00020000);
    const uint32_t koff = (uint32_t)(kb0 + kb) * KBYTES;
    if (d == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rs, LPTR(sas + 64 * sa_grp), 4, saoff,
                                               (uint32_t)((kb0 + kb) * p.ld_sa * 4), 0, 0);
    } else if (d <= C::W_LD) {
      const int i = d - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, LPTR(st + (wave + i * C::WAVES) * 8 * KBYTES), 16, woff[i], koff, 0, 0);
    } else {
      const int i = d - 1 - C::W_LD;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, LPTR(st + C::W_BYTES + (wave + i * C::WAVES) * 8 * KBYTES), 16,
                                               aoff[i], koff, 0, 0);
    }
#endif
  };
  auto issue = [&](int kb, uint8_t* st, float* sas) {
#pragma unroll
    for (int d = 0; d < NPART; ++d) issue_part(kb, st, sas, d);
  };

  // this lane's tokens within the tile (one per m-tile)
  int tok[C::TM];
#pragma unroll
  for (int j = 0; j < C::TM; ++j) tok[j] = wm * (C::BM / C::WM) + j * 16 + (lane & 15);
  const int64_t nb = (n0 + wn * (C::BN / C::WN)) / 128;  // this wave's weight block row

  v4f acc[C::TN][C::TM];
#pragma unroll
  for (int i = 0; i < C::TN; ++i)
#pragma unroll
    for (int j = 0; j < C::TM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // The weight-block scales of the tile's block rows, s_w[n0/128 + b, kb0 .. kb0+KB-1] (either format,
  // decoded to float32), are staged once in LDS (K <= 32768); a step reads its wave's value with
  // one broadcast LDS read.
  constexpr int NBT = C::BN / 128 > 0 ? C::BN / 128 : 1;
  __shared__ __attribute__((aligned(16))) float sws[NBT * 256];
  if constexpr (SCH != 2) {
    for (int idx = tid; idx < NBT * KB; idx += C::THREADS) {
      const int b = idx / KB, k = idx - b * KB;
      sws[b * 256 + k] = load_sw<SWF>(p.s_w, sw_base + (n0 / 128 + b) * KBF + kb0 + k);
    }
    // own LDS writes complete before the first step's barrier (a barrier without a fence)
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  }
  const float* sw_lds = sws + (int)(nb - n0 / 128) * 256;

  // A wave whose token rows all lie past the tile's last row (the last tile of an expert or of
  // M) only issues its copies: its outputs are never stored, and on a SIMD left with one working
  // wave that wave runs alone.  (Two-stage tiles only: with three stages the branch made the
  // compiler wait for the younger copies that the pipeline leaves in flight.)
  const bool active = C::STAGES != 2 || wm * (C::BM / C::WM) < row_end - row0;

  // One K-block of the wave's sub-tile: one MFMA per 16x16 tile gives the partial P, then
  // acc += P * (s_a * s_w).  The MFMAs, the scale-FMAs and the fragment reads are interleaved so
  // that matrix core, VALU and LDS work overlap instead of waiting on each other.
  // The copies of block kb_next go out spread over the first MFMAs, one every SPACING.
  auto compute = [&](const uint8_t* st, const float* sas_cur, const float* swp, int kb_next, uint8_t* refill,
                     float* sas_refill) {
    if (!active) {
#pragma unroll
      for (int d = 0; d < NPART; ++d) issue_part(kb_next, refill, sas_refill, d);
      return;
    }
    const uint8_t* ws = st + wn * (C::BN / C::WN) * KBYTES;
    const uint8_t* as = st + C::W_BYTES + wm * (C::BM / C::WM) * KBYTES;
    if constexpr (SCH == 2) {
      // no per-block factor: every MFMA accumulates into its tile, fragments read in order of
      // first use as below, the copies spread over the MFMAs
      v8i af[2], bf[C::TM];
      af[0] = lds_frag(ws, 0, lane);
#pragma unroll
      for (int j = 0; j < C::TM; ++j) bf[j] = lds_frag(as, j * 16, lane);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int T = C::TN * C::TM;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        {
          constexpr int SP = (NPART - 1) * SPACING < T ? SPACING : (T - 1) / (NPART - 1);
          static_assert(SP >= 1 && (NPART - 1) * SP < T, "copies fit the MFMA sequence");
          if (t % SP == 0 && t / SP < NPART) issue_part(kb_next, refill, sas_refill, t / SP);
        }
        const int i = t / C::TM, j = t % C::TM;
        acc[i][j] = mfma_f8_16x16x128<CODE>(af[i & 1], bf[j], acc[i][j]);
        if (j == 0 && i + 1 < C::TN) af[(i + 1) & 1] = lds_frag(ws, (i + 1) * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    float sc[C::TM];
    {
      // LDS reads in the order of first use (they complete in order, so a wait covers only what
      // the next MFMA needs): the first W fragment and the A fragments, then W fragment i+1 with
      // the first MFMA of W fragment i, the scales with the second MFMA.
      v8i af[2], bf[C::TM];
      af[0] = lds_frag(ws, 0, lane);
#pragma unroll
      for (int j = 0; j < C::TM; ++j) bf[j] = lds_frag(as, j * 16, lane);
      __builtin_amdgcn_sched_barrier(0);
      float sav[C::TM], swv = 0.0f;
      // MFMA t = (i, j) in i-major order; the scale-FMAs of MFMA t - LAG (one W fragment earlier)
      // follow MFMA t, by which time its result is long complete.  The order is pinned: left to
      // itself the scheduler hoists every fragment read to the top, which costs registers and
      // makes the first MFMA wait for all of them.
      constexpr int LAG = C::TM;
      constexpr int T = C::TN * C::TM;
      v4f P[LAG + 1];
#pragma unroll
      for (int t = 0; t < T + LAG; ++t) {
        {
          // every copy issued within the loop (T + LAG iterations)
          constexpr int SP = (NPART - 1) * SPACING < T + LAG ? SPACING : (T + LAG - 1) / (NPART - 1);
          static_assert(SP >= 1 && (NPART - 1) * SP < T + LAG, "copies fit the MFMA sequence");
          if (t % SP == 0 && t / SP < NPART) issue_part(kb_next, refill, sas_refill, t / SP);
        }
        if (t < T) {
          const int i = t / C::TM, j = t % C::TM;
          P[t % (LAG + 1)] = mfma_f8_16x16x128<CODE>(af[i & 1], bf[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
          // fragment i+1 into the buffer whose MFMAs (fragment i-1) are all issued
          if (j == 0 && i + 1 < C::TN) af[(i + 1) & 1] = lds_frag(ws, (i + 1) * 16, lane);
          if (t == 1) {
            if constexpr (SCH == 0) {
#pragma unroll
              for (int jj = 0; jj < C::TM; ++jj) sav[jj] = sas_cur[tok[jj]];
            }
            swv = *swp;
          }
        }
        if (t == LAG) {
#pragma unroll
          for (int j = 0; j < C::TM; ++j) sc[j] = SCH == 0 ? sav[j] * swv : swv;
        }
        if (t >= LAG) {
          const int u = t - LAG;
          acc[u / C::TM][u % C::TM] += P[u % (LAG + 1)] * sc[u % C::TM];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Block kb (tiles and activation scales) lives in stage kb % STAGES.  A step waits for its own
  // block's copies (leaving the younger copies in flight), synchronizes, starts the copies for
  // kb+STAGES-1 into the stage consumed one step earlier, and multiplies block kb.  Past the last
  // block the loads are clamped to it (harmless re-reads into a stage no later step reads), so
  // every step issues the same loads and one fixed vmcnt wait covers all of them.
  auto step = [&](int kb, const uint8_t* cur, const float* sas_cur, uint8_t* refill, float* sas_refill) {
    // own copies of block kb (and its scales) landed, leaving the younger ones in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<C::STAGES == 3 ? C::NDMA : 0>());
    wg_barrier();
    const int kb_next = min(kb + C::STAGES - 1, KB - 1);
    compute(cur, sas_cur, sw_lds + kb, kb_next, refill, sas_refill);
  };

  issue(0, stage0, sas0);
  if (C::STAGES == 3) issue(min(1, KB - 1), stage1, sas1);
  if constexpr (C::STAGES == 2) {
    for (int kb = 0; kb < KB; kb += 2) {
      step(kb, stage0, sas0, stage1, sas1);
      if (kb + 1 < KB) step(kb + 1, stage1, sas1, stage0, sas0);
    }
  } else {
    for (int kb = 0; kb < KB; kb += 3) {
      step(kb, stage0, sas0, stage2, sas2);
      if (kb + 1 < KB) step(kb + 1, stage1, sas1, stage0, sas0);
      if (kb + 2 < KB) step(kb + 2, stage2, sas2, stage1, sas1);
    }
  }
  // The last steps re-issued copies of the final block (clamped) into stages that nothing reads
  // any more; they must have landed before the stages are reused for the output tile below and
  // before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());

  if constexpr (SCH != 0) {
    // scales that do not vary along K: the activation scale of each token (or of the tensor),
    // then, for scheme 2, the channel scale of each output feature
    float ea[C::TM];
#pragma unroll
    for (int j = 0; j < C::TM; ++j) {
      int64_t m = row0 + tok[j];
      m = m < row_end ? m : row_end - 1;
      ea[j] = gload<float>(p.s_a + (p.a_kind == 2 ? 0 : m));
    }
#pragma unroll
    for (int i = 0; i < C::TN; ++i) {
      v4f ew = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (SCH == 2)
        ew = gload<v4f>(reinterpret_cast<const float*>(p.s_w) + n0 + wn * (C::BN / C::WN) + i * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < C::TM; ++j) {
        acc[i][j] = acc[i][j] * ea[j];
        if constexpr (SCH == 2) acc[i][j] = acc[i][j] * ew;
      }
    }
  }

  // epilogue.  bf16 tiles go through LDS in rounds of two 64-row chunks (stage0 and stage1, free
  // once every wave is past its last block) so that the global stores write whole 128-byte
  // lines; stored directly, a lane's 4 consecutive output features of one token make every store
  // instruction touch 16 rows.
  constexpr int ROWB = C::BN * 2 + 16;  // padded LDS row: the 16 rows of a fragment hit distinct banks
  if constexpr (OUT == 0 && C::BM % 128 == 0 && 64 * ROWB <= C::STAGE) {
    constexpr int CPR = C::BN * 2 / 16;  // 16-byte chunks per output row
    // a wave's token rows lie inside one 64-row chunk, so the round and the chunk that take them
    // follow from the wave index alone (a wave-uniform branch: each wave converts its values once)
    static_assert(64 % (C::BM / C::WM) == 0, "a wave's rows stay inside one 64-row chunk");
    const int wrow = wm * (C::BM / C::WM);
#pragma unroll
    for (int r = 0; r < C::BM / 128; ++r) {
      wg_barrier();
      if ((wrow >> 7) == r) {
        uint8_t* const half = (wrow & 64) ? stage1 : stage0;
#pragma unroll
        for (int j = 0; j < C::TM; ++j) {
          const int ml = (wrow & 63) + j * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < C::TN; ++i) {
            const int nl = wn * (C::BN / C::WN) + i * 16 + 4 * (lane >> 4);
            uint2 w;
            w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint2*>(half + ml * ROWB + nl * 2) = w;
          }
        }
      }
      wg_barrier_after_lds_writes();
      for (int c = tid; c < 128 * CPR; c += C::THREADS) {
        const int mr = c / CPR, ch = c - mr * CPR;
        const int64_t m = row0 + r * 128 + mr;
        if (m < row_end) {
          const uint8_t* half = mr < 64 ? stage0 : stage1;
          const v4i v = *reinterpret_cast<const v4i*>(half + (mr & 63) * ROWB + ch * 16);
          // non-temporal: the output streams past the last-level cache, which keeps the operands
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(p.y) + m * p.ldy + n0 + ch * 8));
        }
      }
    }
  } else {
    // lane holds 4 consecutive output features of one token per MFMA tile (K-sliced: into this
    // workgroup's slice of the partial sums)
    void* const ydst = SPLIT ? (void*)(reinterpret_cast<float*>(p.y) + (int64_t)blockIdx.y * p.M * p.ldy) : p.y;
#pragma unroll
    for (int j = 0; j < C::TM; ++j) {
      const int64_t m = row0 + wm * (C::BM / C::WM) + j * 16 + (lane & 15);
      if (m < row_end) {
#pragma unroll
        for (int i = 0; i < C::TN; ++i) {
          const int64_t n = n0 + wn * (C::BN / C::WN) + i * 16 + 4 * (lane >> 4);
          store4<OUT>(ydst, p.ldy, m, n, acc[i][j]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Persistent variant for 256 x 256 tiles when a launch has several tiles per CU (dense or
// grouped, two stages, an even number of K-blocks, bf16 output): one workgroup per CU walks its
// tiles (in the order the one-tile-per-workgroup launch runs them), and the work between two
// tiles is overlapped:
//   * the next tile's first block is copied during the current tile's last step, into the stage
//     that step frees, and its weight-block scales during the current tile's first step, into
//     the scale buffer the current tile does not read;
//   * the output tile is staged through the other stage (free after the last step) in two
//     rounds of 128 token rows, rows swizzled instead of padded (chunk c of row m at c ^ (m & 15));
//   * the stores are range-checked buffer stores (rows past the tile's last row are dropped by
//     the hardware), so every thread issues the same number of them and the next tile's first
//     wait can leave exactly those in flight.
// Per step, the copies and the schedule are those of gemm_prefill_kernel.
// ---------------------------------------------------------------------------------------------
template <typename C, int SWF, bool GROUPED>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_prefill_persistent_kernel(GemmArgs p, int tiles_m,
                                                                                  int tiles_n) {
  static_assert(C::STAGES == 2 && C::BM == 256 && C::BN == 256 && C::WN == 2, "two-stage 256 x 256 tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[C::STAGE];
  __shared__ __attribute__((aligned(16))) float sas0[C::BM];
  __shared__ __attribute__((aligned(16))) float sas1[C::BM];
  // weight-block scales of a tile's two block rows, by tile parity: float32 [2][256], or UE8M0
  // bytes [2][256] in the first 512 bytes
  __shared__ __attribute__((aligned(16))) float swr0[2 * 256];
  __shared__ __attribute__((aligned(16))) float swr1[2 * 256];

  const int64_t K = p.K, M = p.M;
  const int KB = (int)(K / KBYTES);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Grouped (at most 63 experts): lane l holds offsets[l] and the inclusive prefix sum over
  // experts 0..l of their tile-row counts; tiles are numbered expert by expert, and tiles_m (an
  // upper bound) is replaced by the real count.
  int c_off = 0, c_end = 0, c_inc = 0;
  int real_tiles_m = tiles_m;
  if constexpr (GROUPED) {
    // clamped to 0..M, and no tiles for an expert whose end lies before its start (bad offsets
    // then cannot move a tile's rows outside 0..M-1)
    if (p.slot > 0) {  // batched layout: the slot's first row and its count (clamped to the slot)
      c_off = lane < p.E ? lane * (int)p.slot : 0;
      c_end = lane < p.E ? c_off + min(max(gload<int>(p.offsets + lane), 0), (int)p.slot) : 0;
    } else {
      c_off = lane <= p.E ? min(max(gload<int>(p.offsets + lane), 0), (int)M) : 0;
      c_end = __shfl_down(c_off, 1);
    }
    const int nxt = c_end;
    c_inc = lane < p.E && nxt > c_off ? (nxt - c_off + C::BM - 1) / C::BM : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(c_inc, d);
      if (lane >= d) c_inc += t;
    }
    // (never above the host's bound, which valid offsets cannot exceed)
    real_tiles_m = min(__builtin_amdgcn_readfirstlane(__shfl(c_inc, 62)), tiles_m);
  }
  const int ntiles = real_tiles_m * tiles_n;
  if ((int)blockIdx.x >= ntiles) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::WN, wm = wave / C::WN;
  const int lrow = lane >> 3;
  const int GROUP_M = p.K <= 16 * KBYTES ? 4 : 8;
  // this wave's scale copy: float32, block row sw_q / 4, K-block 64 (sw_q % 4) + lane; UE8M0 (K
  // a multiple of 4 blocks), block row sw_q % 2, K-blocks 4 lane .. 4 lane + 3 in one dword
  const int sw_q = wave % 8;

  // A tile is a few uniform values (rows row0 .. row_end-1 of the activations, for grouped those
  // of expert e); its copies address through buffer descriptors based at the tile, so the
  // per-lane offsets below are the same for every tile.  Activation rows past row_end fall outside
  // the descriptors' ranges: their copies are dropped (the rows feed only output rows that are
  // never stored).
  struct Tile {
    int64_t row0, n0, row_end;
    int e;
  };
  auto make_tile = [&](int v) {
    Tile t;
    const int pid = xcd_remap(v, ntiles);
    const int in_group = GROUP_M * tiles_n;
    if constexpr (GROUPED) {
      // Expert e owns tiles tiles_n * (tile-rows before e) onward; inside an expert the tiles
      // run in bands of GROUP_M of its tile-rows, so a band's concurrent tiles share the
      // expert's weight tiles (bands across experts mixed several experts' weights).  The
      // expert is the first lane whose tile prefix reaches past pid (an empty expert's prefix
      // equals the one before it).
      const int first = __builtin_amdgcn_readfirstlane(__ffsll((long long)__ballot(c_inc * tiles_n > pid)) - 1);
      const int before = first > 0 ? __builtin_amdgcn_readlane(c_inc, first - 1) : 0;
      const int mt = __builtin_amdgcn_readlane(c_inc, first) - before;
      const int local = pid - before * tiles_n;
      const int first_m = (local / in_group) * GROUP_M;
      const int gsize = min(mt - first_m, GROUP_M);
      const int pid_m = first_m + (local % in_group) % gsize;
      t.n0 = (int64_t)((local % in_group) / gsize) * C::BN;
      t.e = first;
      t.row0 = (int64_t)__builtin_amdgcn_readlane(c_off, first) + (int64_t)pid_m * C::BM;
      t.row_end = __builtin_amdgcn_readlane(c_end, first);
    } else {
      const int first_m = (pid / in_group) * GROUP_M;
      const int gsize = min(real_tiles_m - first_m, GROUP_M);
      const int pid_m = first_m + (pid % in_group) % gsize;
      t.n0 = (int64_t)((pid % in_group) / gsize) * C::BN;
      t.e = 0;
      t.row0 = (int64_t)pid_m * C::BM;
      t.row_end = M;
    }
    return t;
  };
  uint32_t woff[C::W_LD], aoff[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::W_LD; ++i) {
    const int r = 8 * (wave + i * C::WAVES) + lrow;
    woff[i] = (uint32_t)(r * K + (((lane & 7) ^ swz_g(r)) * 16));
  }
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int r = 8 * (wave + i * C::WAVES) + lrow;
    aoff[i] = (uint32_t)(r * p.lda + (((lane & 7) ^ swz_g(r)) * 16));
  }
  const uint32_t saoff = (uint32_t)((64 * (wave % C::SA_LD) + lane) * 4);
  const uint32_t swoff = SWF == 0 ? (uint32_t)(((sw_q >> 2) * KB + min(64 * (sw_q & 3) + lane, KB - 1)) * 4)
                                  : (uint32_t)((sw_q & 1) * KB + 4 * min(lane, KB / 4 - 1));

  // Copy d of block kb of tile t into stage st: 0 the activation scales, then the weight and
  // activation 8-row groups, and last (a tile's first step only) the weight-block scales of tile
  // ts into swr, the buffer the current tile does not read.
  constexpr int NPART = 2 + C::W_LD + C::A_LD;
  auto issue_part = [&](const Tile t, int kb, uint8_t* st, float* sas, const Tile ts, float* swr, int d) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the builtins exist in the device pass only)
    const uint32_t koff = (uint32_t)kb * KBYTES;
    const uint32_t rows = (uint32_t)(t.row_end - t.row0);
    if (d == 0) {
      // (the K-block goes into the base: the range check then covers exactly the tile's rows)
      const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.s_a + (int64_t)kb * p.ld_sa + t.row0), 0, (int)(rows * 4), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rs, LPTR(sas + 64 * (wave % C::SA_LD)), 4, saoff, 0, 0, 0);
    } else if (d <= C::W_LD) {
      const __amdgpu_buffer_rsrc_t w_rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(p.w_q + ((int64_t)t.e * p.N + t.n0) * K), 0, -1, 0x00020000);
      const int i = d - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rs, LPTR(st + (wave + i * C::WAVES) * 8 * KBYTES), 16, woff[i],
                                               koff, 0, 0);
    } else if (d <= C::W_LD + C::A_LD) {
      const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.a_q + t.row0 * p.lda), 0, (int)(uint32_t)(rows * (uint64_t)p.lda), 0x00020000);
      const int i = d - 1 - C::W_LD;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, LPTR(st + C::W_BYTES + (wave + i * C::WAVES) * 8 * KBYTES), 16,
                                               aoff[i], koff, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t sw_rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const uint8_t*)p.s_w + ((int64_t)ts.e * (p.N / 128) + ts.n0 / 128) * KB * (SWF == 0 ? 4 : 1)), 0,
          -1, 0x00020000);
      uint8_t* const dst = (uint8_t*)swr + (SWF == 0 ? sw_q * 256 : (sw_q & 1) * 256);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sw_rs, LPTR(dst), 4, swoff, 0, 0, 0);
    }
#endif
  };

  int tok[C::TM];
#pragma unroll
  for (int j = 0; j < C::TM; ++j) tok[j] = wm * (C::BM / C::WM) + j * 16 + (lane & 15);
  const int sw_b = wn;  // this wave's weight block row within the tile (128 rows per wave)

  v4f acc[C::TN][C::TM];

  // One K-block (the schedule of gemm_prefill_kernel); the copies of block kn of tile tn, and in
  // a tile's first step (WithSw) the weight-block scales of tile ts, go out spread over the first
  // MFMAs.
  auto compute = [&](auto WithSw, const uint8_t* st, const float* sas_cur, const float* swr_cur, int kb,
                     const Tile tn, int kn, uint8_t* refill, float* sas_refill, const Tile ts, float* swr_next) {
    constexpr int NP = decltype(WithSw)::value ? NPART : NPART - 1;
    const uint8_t* ws = st + wn * (C::BN / C::WN) * KBYTES;
    const uint8_t* as = st + C::W_BYTES + wm * (C::BM / C::WM) * KBYTES;
    float sc[C::TM];
    v8i af[2], bf[C::TM];
    af[0] = lds_frag(ws, 0, lane);
#pragma unroll
    for (int j = 0; j < C::TM; ++j) bf[j] = lds_frag(as, j * 16, lane);
    __builtin_amdgcn_sched_barrier(0);
    float sav[C::TM], swv = 0.0f;
    constexpr int LAG = C::TM;
    constexpr int T = C::TN * C::TM;
    v4f P[LAG + 1];
#pragma unroll
    for (int t = 0; t < T + LAG; ++t) {
      {
        constexpr int SP = (NP - 1) * SPACING < T + LAG ? SPACING : (T + LAG - 1) / (NP - 1);
        static_assert(SP >= 1 && (NP - 1) * SP < T + LAG, "copies fit the MFMA sequence");
        if (t % SP == 0 && t / SP < NP) issue_part(tn, kn, refill, sas_refill, ts, swr_next, t / SP);
      }
      if (t < T) {
        const int i = t / C::TM, j = t % C::TM;
        P[t % (LAG + 1)] = mfma_e4m3_16x16x128(af[i & 1], bf[j]);
        if (j == 0 && i + 1 < C::TN) af[(i + 1) & 1] = lds_frag(ws, (i + 1) * 16, lane);
        if (t == 1) {
#pragma unroll
          for (int jj = 0; jj < C::TM; ++jj) sav[jj] = sas_cur[tok[jj]];
          if constexpr (SWF == 0) swv = swr_cur[sw_b * 256 + kb];
          else swv = dec_ue8m0(reinterpret_cast<const uint8_t*>(swr_cur)[sw_b * 256 + kb]);
        }
      }
      if (t == LAG) {
#pragma unroll
        for (int j = 0; j < C::TM; ++j) sc[j] = sav[j] * swv;
      }
      if (t >= LAG) {
        const int u = t - LAG;
        acc[u / C::TM][u % C::TM] += P[u % (LAG + 1)] * sc[u % C::TM];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // output: y rows past M are out of the descriptor's range and dropped
  constexpr int ROW = C::BN * 2, CPR = ROW / 16;
  constexpr int NSTORE = C::BM * CPR / C::THREADS;  // stores per thread per tile
  auto epilogue = [&](const Tile& t) {
#if defined(__HIP_DEVICE_COMPILE__)
    // the thread index passes through an empty asm so that the addresses below are computed here
    // for each tile rather than hoisted out of the tile loop (where they would be spilled)
    int et = tid;
    asm volatile("" : "+v"(et));
    const int el = et & 63;
    const __amdgpu_buffer_rsrc_t y_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((uint8_t*)p.y + (t.row0 * p.ldy + t.n0) * 2), 0, (int)(uint32_t)((t.row_end - t.row0) * p.ldy * 2), 0x00020000);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      wg_barrier();  // the previous round's reads (and, for r = 0, the last block's) are done
      if (wm / 2 == r) {
#pragma unroll
        for (int j = 0; j < C::TM; ++j) {
          const int mh = (wm % 2) * 64 + j * 16 + (el & 15);
#pragma unroll
          for (int i = 0; i < C::TN; ++i) {
            const int nl = wn * 128 + i * 16 + 4 * (el >> 4);
            uint2 w;
            w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint2*>(stage1 + mh * ROW + (((nl >> 3) ^ (mh & 15)) << 4) + ((nl & 4) << 1)) = w;
          }
        }
      }
      wg_barrier_after_lds_writes();
#pragma unroll
      for (int u = 0; u < NSTORE / 2; ++u) {
        const int c = et + u * C::THREADS;
        const int mh = c / CPR, ch = c - mh * CPR;
        const v4i v = *reinterpret_cast<const v4i*>(stage1 + mh * ROW + ((ch ^ (mh & 15)) << 4));
        const uint32_t off = (uint32_t)(((r * 128 + mh) * p.ldy + ch * 8) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(v, y_rs, off, 0, 2);  // 2: non-temporal, as above
      }
    }
#endif
  };

  // Every step waits for all of its wave's copies except at a tile's first step, which leaves the
  // previous tile's NSTORE output stores (issued after the copies it needs) in flight.  The
  // prologue's copies are waited for before the loop, so that the compiler's view of what is in
  // flight at the loop head is that of the loop's back edge.
  const int G = (int)gridDim.x;
  int v = (int)blockIdx.x;
  Tile tc = make_tile(v);
#pragma unroll
  for (int d = 0; d < NPART; ++d) issue_part(tc, 0, stage0, sas0, tc, swr0, d);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  // One tile; the scale buffers alternate by tile and are named directly (the unrolled pair of
  // calls below), so that the compiler's LDS alias tracking keeps the reads of one free of waits
  // for the copies into the other.
  auto run_tile = [&](const Tile tc, const Tile tn, const float* swr_cur, float* swr_nxt) {
#pragma unroll
    for (int i = 0; i < C::TN; ++i)
#pragma unroll
      for (int j = 0; j < C::TM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // blocks 0 and 1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<NSTORE>());
    wg_barrier();
    compute(std::true_type{}, stage0, sas0, swr_cur, 0, tc, 1, stage1, sas1, tn, swr_nxt);
    {
      const bool last = KB == 2;
      const Tile tt = last ? tn : tc;
      const int kn = last ? 0 : 2;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      wg_barrier();
      compute(std::false_type{}, stage1, sas1, swr_cur, 1, tt, kn, stage0, sas0, tn, swr_nxt);
    }
    // blocks 2 .. KB-1; the last step copies the next tile's block 0
    for (int kb = 2; kb < KB; kb += 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      wg_barrier();
      compute(std::false_type{}, stage0, sas0, swr_cur, kb, tc, kb + 1, stage1, sas1, tn, swr_nxt);
      const bool last = kb + 2 >= KB;
      const Tile tt = last ? tn : tc;
      const int kn = last ? 0 : kb + 2;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      wg_barrier();
      compute(std::false_type{}, stage1, sas1, swr_cur, kb + 1, tt, kn, stage0, sas0, tn, swr_nxt);
    }
    epilogue(tc);
  };
  // past the last tile the next-tile copies repeat the current tile's (harmless)
  for (;;) {
    Tile tn = make_tile(v + G < ntiles ? v + G : v);
    run_tile(tc, tn, swr0, swr1);
    v += G;
    tc = tn;
    if (v >= ntiles) break;
    tn = make_tile(v + G < ntiles ? v + G : v);
    run_tile(tc, tn, swr1, swr0);
    v += G;
    tc = tn;
    if (v >= ntiles) break;
  }
  // the clamped copies past the last tile and the stores complete before the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
}

#ifndef FGB_BIG_CFG
#define FGB_BIG_CFG 256, 256, 2, 4, 1, 2
#endif
#ifndef FGB_HALF_CFG
#define FGB_HALF_CFG 256, 128, 4, 2, 1, 3
#endif
using Big = Cfg<FGB_BIG_CFG>;
using Half = Cfg<FGB_HALF_CFG>;
using Narrow = Cfg<128, 128, 2, 2, 2, 2>;  // N % 256 != 0: 4 waves, wave tile 64 x 64

}  // namespace
}  // namespace fgb
