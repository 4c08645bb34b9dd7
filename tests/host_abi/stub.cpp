// Stand-ins for the HIP runtime and the kernel launchers (see stub.h).
#include <hip/hip_runtime_api.h>
#include <string.h>

#include "../../fine_grained_block_amd/csrc/internal.h"
#include "stub.h"

StubState g_stub = {0, 0, "gfx950:sramecc+:xnack-", 0, 0, "", 0, 0, 0, 0, nullptr, 1u << 20};

hipError_t hipGetDevice(int* d) {
  if (g_stub.get_device_fails) return hipErrorNoDevice;
  *d = g_stub.device;
  return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int dev) {
  (void)dev;
  memset(p, 0, sizeof(*p));
  strncpy(p->gcnArchName, g_stub.arch, sizeof(p->gcnArchName) - 1);
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

namespace fgb {

static hipError_t launched(const char* name) {
  g_stub.launches++;
  g_stub.last = name;
  return g_stub.launch_error ? hipErrorInvalidValue : hipSuccess;
}

static void record(const GemmArgs& a) {
  g_stub.M = a.M;
  g_stub.N = a.N;
  g_stub.K = a.K;
  g_stub.E = a.E;
}

hipError_t launch_act_quant(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                            hipStream_t) {
  return launched("act_quant");
}
hipError_t launch_weight_quant(const uint16_t*, int64_t, int64_t, uint8_t*, void*, int, hipStream_t, int) {
  return launched("weight_quant");
}
hipError_t launch_row_quant(const uint16_t*, int64_t rows, int64_t K, int64_t, uint8_t*, int64_t, float*, int,
                            hipStream_t) {
  g_stub.M = rows;
  g_stub.K = K;
  return launched("row_quant");
}
hipError_t launch_static_quant(const uint16_t*, int64_t, int64_t, int64_t, const float*, uint8_t*, int64_t, int,
                               hipStream_t) {
  return launched("static_quant");
}
hipError_t launch_gemm_scaled_prefill(const GemmArgs& a, int sch, int, hipStream_t) {
  record(a);
  g_stub.E = sch;
  return launched("scaled_prefill");
}
hipError_t launch_gemm_scaled_decode(const GemmArgs& a, int sch, int, void* ws, hipStream_t) {
  record(a);
  g_stub.E = sch;
  g_stub.workspace = ws;
  return launched("scaled_decode");
}
hipError_t launch_encode(const float*, uint8_t*, int64_t, int, int, hipStream_t) { return launched("encode"); }
hipError_t launch_decode(const uint8_t*, float*, int64_t, int, hipStream_t) { return launched("decode"); }
hipError_t launch_selftest_quotients(unsigned long long*, hipStream_t) { return launched("selftest"); }
hipError_t launch_gemm_prefill(const GemmArgs& a, void* ws, hipStream_t) {
  record(a);
  g_stub.workspace = ws;
  return launched("gemm_prefill");
}
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return (M == 256 && N == 4096 && K == 4096) ? (size_t)g_stub.prefill_ws_query : 0;
}
hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t) {
  record(a);
  return launched("gemm_grouped");
}
hipError_t launch_check_offsets(const int32_t*, int32_t, int64_t, int32_t*, hipStream_t) {
  return launched("check_offsets");
}
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return (M == 32 && N == 4096 && K == 4096) ? (size_t)g_stub.ws_bytes_query : 0;
}
size_t fused_workspace_bytes(int64_t M, int64_t, int64_t) { return M > 8 ? 4096 : 0; }
hipError_t launch_gemm_decode_fused(const GemmArgs& a, const uint16_t*, int64_t, void* ws, hipStream_t) {
  record(a);
  g_stub.workspace = ws;
  return launched("gemm_fused");
}
int decode_small_waves(int64_t, int64_t) { return 8; }
hipError_t launch_gemm_moe_decode(const GemmArgs& a, int mode, hipStream_t) {
  record(a);
  g_stub.K = mode;  // (the driver checks which layout reached the launcher)
  return launched("moe_decode");
}
hipError_t scratch_address(void** out) {
  *out = (void*)0x200000;  // stands for the library's scratch address
  return hipSuccess;
}
hipError_t launch_gemm_decode(const GemmArgs& a, void* ws, hipStream_t) {
  record(a);
  g_stub.workspace = ws;
  return launched("gemm_decode");
}

}  // namespace fgb
