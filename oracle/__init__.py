"""CPU oracle for fine-grained FP8 W8A8 block quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct numpy statement of
what the GPU library computes.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import it; the library itself never does, and it shares no code with the HIP
kernels or their host code.  The one module both sides use is `workloads`, which draws the
seeded synthetic inputs and holds none of the method's arithmetic.

Modules
-------
fp8        E4M3 / E5M2 / UE8M0 decode and encode from the bit fields (float64, exact)
blockquant act_quant (dynamic 1x128 groups), weight_quant (128x128 blocks, float32 or UE8M0)
gemm       gemm_ref (exact per-block partials, float64), gemm_ref_fast, grouped_ref,
           batched_ref (masked [E, max_M] expert slots), bf16_rne
schemes    per-token / per-channel (FP8_DYNAMIC) and static per-tensor quantization, E5M2 codes,
           and the GEMM under those scales (scaled_gemm_ref)

Pins (see tests/test_oracle_*.py): exhaustive code tables against the formats' printed maxima
and NaN/inf sets and against torch's float8 dtypes; brute-force nearest-code searches for the
encoders; closed forms for UE8M0; quantization invariants; hand-worked golden fixtures; a dense
float64 brute force and an exact-integer special case for the GEMM.  Parity unpinned: none of
the functions above; the GEMM's float32 summation order on the GPU is held to a tolerance.
"""
from . import fp8, blockquant, gemm, schemes  # noqa: F401
from .fp8 import dec_e4m3, dec_e5m2, dec_ue8m0, enc_e4m3_sat, enc_e5m2, ue8m0_from_amax  # noqa: F401
from .blockquant import act_quant, weight_quant  # noqa: F401
from .gemm import gemm_ref, gemm_ref_fast, grouped_ref, batched_ref, bf16_rne  # noqa: F401
