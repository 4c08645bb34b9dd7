// Calls every entry point of include/fgb.h with invalid and valid arguments against the host
// stand-ins of stub.cpp; built with AddressSanitizer and UBSan by tests/test_abi_sanitized.py.
// Exits nonzero on the first unexpected status (and the sanitizers abort on any memory error
// or undefined behaviour in the validation code).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/fgb.h"
#include "stub.h"

static int failures = 0;
#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    int got_ = (call);                                                                        \
    if (got_ != (want)) {                                                                     \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
              (int)(want));                                                                   \
      failures++;                                                                             \
    }                                                                                         \
  } while (0)

static void* P(uintptr_t v) { return (void*)v; }
static const uintptr_t F = 0x10000;  // a 16-byte aligned address that is never dereferenced

static int gemm(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ld_sa, int64_t ldy, int fmt = 0, int ydt = 0,
                uintptr_t a = F, uintptr_t ws = 0, size_t wsb = 0) {
  return fgb_w8a8_block_gemm((const uint8_t*)P(a), lda, (const float*)P(F), ld_sa, (const uint8_t*)P(F), P(F), fmt,
                             P(F), ydt, ldy, M, N, K, P(ws), wsb, nullptr);
}

int main() {
  // status strings and version
  for (int s = 0; s >= -8; --s)
    if (!fgb_status_string(s) || strncmp(fgb_status_string(s), "FGB_", 4) != 0) failures++;
  if (strcmp(fgb_status_string(77), "unknown fgb status") != 0) failures++;
  EXPECT(fgb_abi_version(), FGB_ABI_VERSION);

  // GEMM validation
  EXPECT(gemm(256, 512, 1000, 1008, 256, 512), FGB_ERR_SHAPE);
  EXPECT(gemm(256, 500, 1024, 1024, 256, 512), FGB_ERR_SHAPE);
  EXPECT(gemm(-1, 512, 1024, 1024, 256, 512), FGB_ERR_SHAPE);
  EXPECT(gemm((int64_t)1 << 40, 512, 1024, 1024, 256, 512), FGB_ERR_SHAPE);
  EXPECT(gemm(0, 512, 1024, 1024, 256, 512), FGB_OK);
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512, 2), FGB_ERR_ENUM);
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512, 0, 5), FGB_ERR_ENUM);
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512, 0, 0, 0), FGB_ERR_NULL);
  EXPECT(gemm(256, 512, 1024, 512, 256, 512), FGB_ERR_STRIDE);
  EXPECT(gemm(256, 512, 1024, 1024, 100, 512), FGB_ERR_STRIDE);
  EXPECT(gemm(256, 512, 1024, 1024, 256, 256), FGB_ERR_STRIDE);
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512, 0, 0, F + 8), FGB_ERR_ALIGN);
  EXPECT(gemm(256, 512, 1024, 1032, 256, 512), FGB_ERR_ALIGN);
  EXPECT(gemm(256, 512, 1024, 1024, 258, 512), FGB_ERR_ALIGN);
  EXPECT(gemm(256, 512, 65536, 65536, 256, 512), FGB_ERR_SHAPE);       // K above 32768
  EXPECT(gemm(65536, 512, 1024, 65536, 65536, 512), FGB_ERR_SHAPE);    // A beyond 32-bit offsets
  // valid prefill call reaches the prefill launcher with the sizes given
  g_stub.launches = 0;
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512), FGB_OK);
  if (g_stub.launches != 1 || strcmp(g_stub.last, "gemm_prefill") || g_stub.M != 256 || g_stub.N != 512 ||
      g_stub.K != 1024)
    failures++;
  // decode: M <= 64; a workspace is required when the plan asks for one
  EXPECT(gemm(32, 4096, 4096, 4096, 32, 4096), FGB_ERR_WORKSPACE);
  EXPECT(gemm(32, 4096, 4096, 4096, 32, 4096, 0, 0, F, F, (1u << 20) - 1), FGB_ERR_WORKSPACE);
  EXPECT(gemm(32, 4096, 4096, 4096, 32, 4096, 0, 0, F, F + 4, 1u << 20), FGB_ERR_ALIGN);
  EXPECT(gemm(32, 4096, 4096, 4096, 32, 4096, 0, 0, F, F, 1u << 20), FGB_OK);
  if (strcmp(g_stub.last, "gemm_decode") || g_stub.workspace != P(F)) failures++;
  EXPECT(gemm(8, 4096, 4096, 4096, 8, 4096), FGB_OK);
  EXPECT(fgb_gemm_workspace_bytes(65, 4096, 4096), 0);
  EXPECT(fgb_gemm_workspace_bytes(32, 4096, 4096) > 0, 1);
  // prefill with K slices: the plan's workspace is required as well
  g_stub.prefill_ws_query = 8u << 20;
  EXPECT(fgb_gemm_workspace_bytes(256, 4096, 4096), (size_t)8 << 20);
  EXPECT(gemm(256, 4096, 4096, 4096, 256, 4096), FGB_ERR_WORKSPACE);
  EXPECT(gemm(256, 4096, 4096, 4096, 256, 4096, 0, 0, F, F, (8u << 20) - 16), FGB_ERR_WORKSPACE);
  EXPECT(gemm(256, 4096, 4096, 4096, 256, 4096, 0, 0, F, F + 4, 8u << 20), FGB_ERR_ALIGN);
  EXPECT(gemm(256, 4096, 4096, 4096, 256, 4096, 0, 0, F, F, 8u << 20), FGB_OK);
  if (strcmp(g_stub.last, "gemm_prefill") || g_stub.workspace != P(F)) failures++;
  // the no-allocation variant: no workspace argument; decode calls get the library's scratch
  auto noalloc = [](int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ld_sa, int64_t ldy) {
    return fgb_w8a8_block_gemm_noalloc((const uint8_t*)P(F), lda, (const float*)P(F), ld_sa, (const uint8_t*)P(F),
                                       P(F), 0, P(F), 0, ldy, M, N, K, nullptr);
  };
  EXPECT(noalloc(32, 4096, 4096, 4096, 32, 4096), FGB_OK);
  if (strcmp(g_stub.last, "gemm_decode") || g_stub.workspace != P(0x200000)) failures++;
  EXPECT(noalloc(256, 512, 1024, 1024, 256, 512), FGB_OK);
  if (strcmp(g_stub.last, "gemm_prefill")) failures++;
  if (g_stub.workspace != nullptr) failures++;  // no workspace needed: none passed
  EXPECT(noalloc(256, 4096, 4096, 4096, 256, 4096), FGB_OK);  // K-sliced prefill: the scratch
  if (strcmp(g_stub.last, "gemm_prefill") || g_stub.workspace != P(0x200000)) failures++;
  EXPECT(noalloc(8, 4096, 4096, 4096, 8, 4096), FGB_OK);
  if (g_stub.workspace != nullptr) failures++;  // no workspace needed: none passed
  g_stub.ws_bytes_query = (uint64_t)33 << 20;   // a plan beyond the 32 MiB scratch
  EXPECT(noalloc(32, 4096, 4096, 4096, 32, 4096), FGB_ERR_WORKSPACE);
  g_stub.ws_bytes_query = 1u << 20;
  EXPECT(noalloc(32, 4096, 4096, 4096, 16, 4096), FGB_ERR_STRIDE);
  // launch failure and device checks
  g_stub.launch_error = 1;
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512), FGB_ERR_LAUNCH);
  g_stub.launch_error = 0;
  g_stub.get_device_fails = 1;
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512), FGB_ERR_DEVICE);
  g_stub.get_device_fails = 0;
  g_stub.device = 1;
  g_stub.arch = "gfx942:sramecc+:xnack-";
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512), FGB_ERR_DEVICE);
  g_stub.device = 70;  // beyond the library's device table
  EXPECT(gemm(256, 512, 1024, 1024, 256, 512), FGB_ERR_DEVICE);
  g_stub.device = 0;
  g_stub.arch = "gfx950:sramecc+:xnack-";

  // grouped GEMM
  auto grouped = [](int32_t E, int64_t tM, uintptr_t off, int64_t N = 512) {
    return fgb_grouped_w8a8_block_gemm((const uint8_t*)P(F), 1024, (const float*)P(F), 256, (const uint8_t*)P(F),
                                       P(F), 0, (const int32_t*)P(off), E, tM, P(F), 0, 512, N, 1024, nullptr, 0,
                                       nullptr);
  };
  EXPECT(grouped(0, 256, F), FGB_ERR_SHAPE);
  EXPECT(grouped(65536, 256, F), FGB_ERR_SHAPE);
  EXPECT(grouped(4, 256, 0), FGB_ERR_NULL);
  EXPECT(grouped(4, 256, F + 2), FGB_ERR_ALIGN);
  EXPECT(grouped(4, 0, F), FGB_OK);
  EXPECT(grouped(4, 256, F, 100), FGB_ERR_SHAPE);
  EXPECT(grouped(4, 256, F), FGB_OK);
  if (strcmp(g_stub.last, "gemm_grouped") || g_stub.E != 4 || g_stub.M != 256) failures++;
  EXPECT(grouped(4, 64, F), FGB_OK);  // at most 64 rows in all: the per-expert decode kernel
  if (strcmp(g_stub.last, "moe_decode") || g_stub.K != 1) failures++;
  auto batched = [](int32_t E, int64_t max_m, uintptr_t cnt, int64_t ld_sa = 4096) {
    return fgb_batched_w8a8_block_gemm((const uint8_t*)P(F), 1024, (const float*)P(F), ld_sa, (const uint8_t*)P(F),
                                       P(F), 0, (const int32_t*)P(cnt), E, max_m, P(F), 0, 512, 512, 1024, nullptr);
  };
  EXPECT(batched(0, 64, F), FGB_ERR_SHAPE);
  EXPECT(batched(65536, 0, F), FGB_ERR_SHAPE);
  EXPECT(batched(8, -1, F), FGB_ERR_SHAPE);
  EXPECT(batched(8, 64, 0), FGB_ERR_NULL);
  EXPECT(batched(8, 64, F + 2), FGB_ERR_ALIGN);
  EXPECT(batched(8, 64, F, 500), FGB_ERR_STRIDE);  // ld_sa below E * max_M
  EXPECT(batched(8, 0, F), FGB_OK);
  EXPECT(batched(8, 64, F), FGB_OK);
  if (strcmp(g_stub.last, "moe_decode") || g_stub.K != 2 || g_stub.M != 512) failures++;
  EXPECT(batched(8, 256, F), FGB_OK);
  if (strcmp(g_stub.last, "gemm_grouped") || g_stub.M != 2048) failures++;
  EXPECT(fgb_grouped_gemm_workspace_bytes(256, 512, 1024, 4), 0);

  // quantizers and codecs
  EXPECT(fgb_act_quant_group128((const uint16_t*)P(F), 64, 1000, 1000, (uint8_t*)P(F), 1008, (float*)P(F), 64,
                                nullptr), FGB_ERR_SHAPE);
  EXPECT(fgb_act_quant_group128(nullptr, 64, 1024, 1024, (uint8_t*)P(F), 1024, (float*)P(F), 64, nullptr),
         FGB_ERR_NULL);
  EXPECT(fgb_act_quant_group128((const uint16_t*)P(F), 64, 1024, 1024, (uint8_t*)P(F), 1024, (float*)P(F), 32,
                                nullptr), FGB_ERR_STRIDE);
  EXPECT(fgb_act_quant_group128((const uint16_t*)P(F), 64, 1024, 1028, (uint8_t*)P(F), 1024, (float*)P(F), 64,
                                nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_act_quant_group128((const uint16_t*)P(F), 64, 1024, 1024, (uint8_t*)P(F), 1024, (float*)P(F), 64,
                                nullptr), FGB_OK);
  EXPECT(fgb_weight_quant_block128((const uint16_t*)P(F), 130, 128, (uint8_t*)P(F), P(F), 0, nullptr), FGB_ERR_SHAPE);
  EXPECT(fgb_weight_quant_block128((const uint16_t*)P(F), 128, 128, (uint8_t*)P(F), P(F), 9, nullptr), FGB_ERR_ENUM);
  EXPECT(fgb_weight_quant_block128((const uint16_t*)P(F), 128, 128, (uint8_t*)P(F), P(F + 1), 0, nullptr),
         FGB_ERR_ALIGN);
  EXPECT(fgb_weight_quant_block128((const uint16_t*)P(F), 128, 128, (uint8_t*)P(F), P(F + 1), 1, nullptr), FGB_OK);
  EXPECT(fgb_fp8_encode((const float*)P(F), (uint8_t*)P(F), 16, 9, 1, nullptr), FGB_ERR_ENUM);
  EXPECT(fgb_fp8_encode((const float*)P(F), (uint8_t*)P(F), -1, 0, 1, nullptr), FGB_ERR_SHAPE);
  EXPECT(fgb_fp8_encode((const float*)P(F), (uint8_t*)P(F), 16, 0, 1, nullptr), FGB_OK);
  EXPECT(fgb_fp8_decode((const uint8_t*)P(F), (float*)P(F + 1), 16, 0, nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_fp8_decode((const uint8_t*)P(F), (float*)P(F), 16, 3, nullptr), FGB_ERR_ENUM);
  EXPECT(fgb_fp8_decode((const uint8_t*)P(F), (float*)P(F), 16, 2, nullptr), FGB_OK);
  EXPECT(fgb_check_expert_offsets((const int32_t*)P(F), 0, 10, (int32_t*)P(F), nullptr), FGB_ERR_SHAPE);
  EXPECT(fgb_check_expert_offsets((const int32_t*)P(F), 4, 10, (int32_t*)P(F + 1), nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_check_expert_offsets((const int32_t*)P(F), 4, 10, (int32_t*)P(F), nullptr), FGB_OK);
  EXPECT(fgb_selftest_quotients(nullptr, nullptr), FGB_ERR_NULL);
  EXPECT(fgb_selftest_quotients((unsigned long long*)P(F + 4), nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_selftest_quotients((unsigned long long*)P(F), nullptr), FGB_OK);

  // the other schemes: per-token / per-channel / static quantizers and the scaled GEMM
  EXPECT(fgb_act_quant_per_token((const uint16_t*)P(F), 64, 1024, 1024, 7, (uint8_t*)P(F), 1024, (float*)P(F),
                                 nullptr), FGB_ERR_ENUM);
  EXPECT(fgb_act_quant_per_token((const uint16_t*)P(F), 64, 1000, 1000, 0, (uint8_t*)P(F), 1008, (float*)P(F),
                                 nullptr), FGB_ERR_SHAPE);
  EXPECT(fgb_act_quant_per_token((const uint16_t*)P(F), 64, 1024, 1024, 1, (uint8_t*)P(F), 1024, (float*)P(F + 2),
                                 nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_act_quant_per_token((const uint16_t*)P(F), 64, 1024, 512, 1, (uint8_t*)P(F), 1024, (float*)P(F),
                                 nullptr), FGB_ERR_STRIDE);
  EXPECT(fgb_act_quant_per_token((const uint16_t*)P(F), 64, 1024, 1024, 1, (uint8_t*)P(F), 1024, (float*)P(F + 4),
                                 nullptr), FGB_OK);
  if (strcmp(g_stub.last, "row_quant") || g_stub.M != 64 || g_stub.K != 1024) failures++;
  EXPECT(fgb_weight_quant_per_channel((const uint16_t*)P(F), 200, 1024, 0, (uint8_t*)P(F), (float*)P(F), nullptr),
         FGB_ERR_SHAPE);
  EXPECT(fgb_weight_quant_per_channel((const uint16_t*)P(F), 256, 1024, 0, (uint8_t*)P(F), (float*)P(F), nullptr),
         FGB_OK);
  EXPECT(fgb_act_quant_static((const uint16_t*)P(F), 64, 1024, 1024, nullptr, 0, (uint8_t*)P(F), 1024, nullptr),
         FGB_ERR_NULL);
  EXPECT(fgb_act_quant_static((const uint16_t*)P(F), 64, 1024, 1024, (const float*)P(F + 1), 0, (uint8_t*)P(F),
                              1024, nullptr), FGB_ERR_ALIGN);
  EXPECT(fgb_act_quant_static((const uint16_t*)P(F), 64, 1024, 1024, (const float*)P(F + 4), 1, (uint8_t*)P(F),
                              1024, nullptr), FGB_OK);
  EXPECT(fgb_weight_quant_block128_ex((const uint16_t*)P(F), 128, 128, 1, (uint8_t*)P(F), P(F), 1, nullptr),
         FGB_ERR_ENUM);  // UE8M0 scales go with E4M3 codes
  EXPECT(fgb_weight_quant_block128_ex((const uint16_t*)P(F), 128, 128, 1, (uint8_t*)P(F), P(F), 0, nullptr), FGB_OK);
  auto scaled = [](int64_t M, int ak, int wk, int swf, int code, uintptr_t sa = F + 4, uintptr_t sw = F,
                   int64_t N = 512, int64_t K = 1024, uintptr_t ws = 0, size_t wsb = 0) {
    return fgb_w8a8_scaled_gemm((const uint8_t*)P(F), K, (const float*)P(sa), ak, (const uint8_t*)P(F), P(sw), wk,
                                swf, code, P(F), 0, N, M, N, K, P(ws), wsb, nullptr);
  };
  EXPECT(scaled(256, FGB_ACT_SCALE_GROUP128, FGB_W_SCALE_BLOCK128, 0, 0), FGB_ERR_ENUM);
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, 5, 0, 0), FGB_ERR_ENUM);
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 1, 0), FGB_ERR_ENUM);   // UE8M0 per channel
  EXPECT(scaled(256, FGB_ACT_SCALE_TENSOR, FGB_W_SCALE_BLOCK128, 1, 1), FGB_ERR_ENUM);  // UE8M0 with E5M2
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 3), FGB_ERR_ENUM);
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 2), FGB_ERR_ALIGN);
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 4, F + 4), FGB_ERR_ALIGN);
  EXPECT(scaled(0, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0), FGB_OK);
  EXPECT(scaled(256, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 1), FGB_OK);
  if (strcmp(g_stub.last, "scaled_prefill") || g_stub.E != 2 || g_stub.M != 256) failures++;
  EXPECT(scaled(64, FGB_ACT_SCALE_TENSOR, FGB_W_SCALE_BLOCK128, 1, 0), FGB_OK);
  if (strcmp(g_stub.last, "scaled_decode") || g_stub.E != 1) failures++;
  // a decode plan with partials (the stub's plan for 32 x 4096 x 4096) needs the workspace
  const size_t need = fgb_gemm_workspace_bytes(32, 4096, 4096);
  EXPECT(scaled(32, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 4, F, 4096, 4096), FGB_ERR_WORKSPACE);
  EXPECT(scaled(32, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 4, F, 4096, 4096, F, need - 1), FGB_ERR_WORKSPACE);
  EXPECT(scaled(32, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 4, F, 4096, 4096, F + 8, need), FGB_ERR_ALIGN);
  EXPECT(scaled(32, FGB_ACT_SCALE_TOKEN, FGB_W_SCALE_CHANNEL, 0, 0, F + 4, F, 4096, 4096, F, need), FGB_OK);
  if (strcmp(g_stub.last, "scaled_decode") || g_stub.workspace != P(F)) failures++;

  // the fused-quantization decode GEMM (the stub's workspace need: 4096 bytes above 8 rows)
  auto fused = [](int64_t M, int64_t ldx, uintptr_t xp = F, uintptr_t ws = F, size_t ws_bytes = 4096) {
    return fgb_w8a8_block_gemm_fused_quant((const uint16_t*)P(xp), ldx, (const uint8_t*)P(F), P(F), 0, P(F), 0, 512,
                                           M, 512, 1024, P(ws), ws_bytes, nullptr);
  };
  EXPECT(fused(65, 1024), FGB_ERR_SHAPE);
  EXPECT(fused(16, 1000), FGB_ERR_STRIDE);
  EXPECT(fused(16, 1028), FGB_ERR_ALIGN);
  EXPECT(fused(16, 1024, F + 2), FGB_ERR_ALIGN);
  EXPECT(fused(16, 1024, 0), FGB_ERR_NULL);
  EXPECT(fused(0, 1024), FGB_OK);
  EXPECT(fused(64, 1024, F, 0, 0), FGB_ERR_WORKSPACE);
  EXPECT(fused(64, 1024, F, F, 4095), FGB_ERR_WORKSPACE);
  EXPECT(fused(64, 1024, F, F + 8, 4096), FGB_ERR_ALIGN);
  EXPECT(fused(64, 1024), FGB_OK);
  if (strcmp(g_stub.last, "gemm_fused") || g_stub.M != 64 || g_stub.workspace != P(F)) failures++;
  EXPECT(fused(4, 1024, F, 0, 0), FGB_OK);  // one launch: no workspace needed
  if (strcmp(g_stub.last, "gemm_fused") || g_stub.M != 4) failures++;

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
