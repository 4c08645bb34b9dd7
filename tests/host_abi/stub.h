// Host-only stand-ins for the HIP runtime calls and kernel launchers that the C-ABI code uses,
// so that its validation can be built with g++ under AddressSanitizer and UBSan on a machine
// without a GPU.  The stand-ins record what reached them.
#pragma once
#include <stdint.h>

struct StubState {
  int device;           // what hipGetDevice reports
  int get_device_fails; // hipGetDevice returns an error
  const char* arch;     // gcnArchName of every device
  int launch_error;     // launchers return an error
  int launches;         // launcher calls so far
  const char* last;     // name of the last launcher called
  int64_t M, N, K, E;   // sizes the last GEMM launcher received
  const void* workspace;
  uint64_t ws_bytes_query;  // what decode_workspace_bytes returns for (32, 4096, 4096)
  uint64_t prefill_ws_query;  // what prefill_workspace_bytes returns for (256, 4096, 4096)
};
extern StubState g_stub;
