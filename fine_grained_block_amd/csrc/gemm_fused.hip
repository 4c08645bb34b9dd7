// gemm_fused.hip — act_quant_group128 + w8a8_block_gemm from bf16 activations at decode sizes
// (M <= 64) behind one call.
//
// Few tokens: one launch of the GEMM that quantizes its activations itself
// (gemm_decode_fused_quant_small_kernel).  Every workgroup quantizes the rows it multiplies, so
// the quantization is repeated N/16 times.  Measured against act_quant + GEMM (graph loop, the six
// decode shapes from 4096x4096 to 7168x18432, M = 1 ... 64): the one launch is faster up to 4
// rows where K >= 4096 (4096x4096 6.6-7.0 vs 8.6-9.0 us, 4096x14336 13.2-13.9 vs 15.5-15.9 us)
// and up to 8 rows for weights of at most 16 MiB (4096x4096 8.2 vs 9.3 us at M = 8); with short
// rows (24576x1536) or more rows the separate quantization costs less (6144x4096 at M = 8 11.5 vs
// 10.9 us; 28672x4096 at M = 64 239 vs 33 us with an earlier 16-64-row fused kernel).  Beyond
// those sizes the call quantizes into the caller's workspace and runs the decode GEMM on it: the
// same kernels as the two calls, so the same bits.
#include "gemm_decode_kernels.hpp"

namespace fgb {

namespace {

bool one_launch(int64_t M, int64_t N, int64_t K) { return (M <= 4 && K >= 4096) || (M <= 8 && N * K <= (16ll << 20)); }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// workspace layout: codes [M, K], scales [K/128, ld_sa] with ld_sa = M rounded up to 4 (16-byte
// rows), then the decode GEMM's own workspace
int64_t fused_ld_sa(int64_t M) { return (M + 3) & ~(int64_t)3; }

}  // namespace

size_t fused_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (one_launch(M, N, K)) return 0;
  return round256((size_t)(M * K)) + round256((size_t)((K / 128) * fused_ld_sa(M) * 4)) +
         decode_workspace_bytes(M, N, K);
}

hipError_t launch_gemm_decode_fused(const GemmArgs& a, const uint16_t* x, int64_t ldx, void* workspace,
                                    hipStream_t stream) {
  if (one_launch(a.M, a.N, a.K)) return launch_gemm_decode_fused_small(a, x, ldx, stream);
  uint8_t* q = reinterpret_cast<uint8_t*>(workspace);
  const int64_t ld_sa = fused_ld_sa(a.M);
  float* s_a = reinterpret_cast<float*>(q + round256((size_t)(a.M * a.K)));
  void* ws = reinterpret_cast<uint8_t*>(s_a) + round256((size_t)((a.K / 128) * ld_sa * 4));
  hipError_t e = launch_act_quant(x, a.M, a.K, ldx, q, a.K, s_a, ld_sa, stream);
  if (e != hipSuccess) return e;
  GemmArgs b = a;
  b.a_q = q;
  b.lda = a.K;
  b.s_a = s_a;
  b.ld_sa = ld_sa;
  return launch_gemm_decode(b, ws, stream);
}

}  // namespace fgb
