"""fine_grained_block_amd — fine-grained FP8 W8A8 block quantization and GEMM on MI355X (gfx950).

A thin Python binding over the C-ABI library ``libfgb.so`` (declared in ``include/fgb.h``).
This layer only marshals arguments: it allocates outputs and workspaces with torch (device
memory and the current stream are the only things torch provides) and calls the library; every
step of the computation runs in the library's HIP kernels.  There is no CPU or PyTorch
fallback: if the library is missing, or a call returns a nonzero status, an exception is raised.

    q, s_a = quantize(x)                 # x bf16 [M, K] -> E4M3 codes [M, K], scales [K/128, ld]
    w_q, s_w = quantize_weight(w, "ue8m0")
    y = gemm(q, s_a, w_q, s_w)           # bf16 [M, N]
    y = grouped_gemm(q, s_a, w_q, s_w, offsets)
"""
from ._lib import (  # noqa: F401
    FGBError,
    SCALE_F32,
    SCALE_UE8M0,
    OUT_BF16,
    OUT_F32,
    FP8_E4M3,
    FP8_E5M2,
    UE8M0,
    FP8_E4M3_INT,
    ACT_SCALE_TOKEN,
    ACT_SCALE_TENSOR,
    W_SCALE_BLOCK128,
    W_SCALE_CHANNEL,
    lib,
    lib_path,
    status_string,
)
from .ops import (  # noqa: F401
    quantize,
    quantize_weight,
    quantize_per_token,
    quantize_weight_per_channel,
    quantize_static,
    scaled_gemm,
    gemm,
    gemm_noalloc,
    gemm_fused_quant,
    gemm_fused_quant_workspace_bytes,
    grouped_gemm,
    batched_gemm,
    check_offsets,
    gemm_workspace_bytes,
    fp8_encode,
    fp8_decode,
    linear,
    selftest_quotients,
)
