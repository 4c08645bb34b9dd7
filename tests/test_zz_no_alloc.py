"""GPU: the no-allocation GEMM entry point (fgb_w8a8_block_gemm_noalloc) against the existing
entry point (fgb_w8a8_block_gemm, given a workspace) and the oracle, through the C-ABI.

Two workspace-needing decode calls in a row, the second with a smaller plan, a K-sliced prefill
call, calls that need no scratch (M <= 16, 24 rows on 2-wave workgroups), and 100 rows on the
128-row decode kernel with K slices; the library's scratch keeps the previous call's contents,
which must not matter.  Same kernels, so the outputs are equal bit for bit; both are also held
to the oracle's tolerance."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from oracle import gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, upload

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    rng = np.random.default_rng(seed)
    wq = rng.choice(finite, size=(N, K))
    sw = (rng.uniform(0.25, 4.0, size=(N // 128, K // 128)) / 448).astype(np.float32)
    aq = rng.choice(finite, size=(M, K))
    sa = (rng.uniform(0.25, 4.0, size=(M, K // 128)) / 448).astype(np.float32)
    return aq, sa, wq, sw


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry(dev, out_dtype):
    # (64, 6144, 4096): 5 K slices, 7.9 MB of partials; (40, 1024, 16512): 15 slices, 2.4 MB;
    # then a K-sliced prefill call (2 slices, in the scratch), calls that use no scratch (M <= 16,
    # and 24 rows over 32 K-blocks on 2-wave workgroups over the whole K), and 100 rows on the
    # 128-row decode kernel with 4 K slices
    shapes = [(64, 6144, 4096), (40, 1024, 16512), (300, 1024, 1024), (8, 2048, 2048), (24, 6144, 4096),
              (100, 2048, 4096)]
    assert fgb.gemm_workspace_bytes(*shapes[4]) == 0
    assert fgb.gemm_workspace_bytes(*shapes[0]) > fgb.gemm_workspace_bytes(*shapes[1]) > 0
    for i, (M, N, K) in enumerate(shapes):
        ops = _operands(M, N, K, 500 + i)
        aq, sa, wq, sw = upload(*ops, dev)
        ref_out = fgb.gemm(aq, sa, wq, sw, out_dtype=out_dtype)
        out = torch.full((M, N), float("nan"), dtype=out_dtype, device=dev)
        fgb.gemm_noalloc(aq, sa, wq, sw, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out_dtype == torch.bfloat16 else out.view(torch.int32),
                           ref_out.view(torch.int16) if out_dtype == torch.bfloat16 else ref_out.view(torch.int32))
        yref = gemm.gemm_ref_fast(*ops)
        if out_dtype == torch.float32:
            check_t1(out.cpu().numpy(), yref)
        else:
            check_t2(bf16_tensor_to_f64(out), yref)


def test_noalloc_rejects_missing_output(dev):
    aq, sa, wq, sw = upload(*_operands(16, 256, 256, 9), dev)
    with pytest.raises(ValueError):
        fgb.gemm_noalloc(aq, sa, wq, sw, None)
