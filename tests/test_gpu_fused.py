"""GPU: act_quant_group128 + w8a8_block_gemm from bf16 activations in one call
(fgb_w8a8_block_gemm_fused_quant) against the two-launch path and the oracle, through the C-ABI.

A few tokens run one launch whose GEMM quantizes the activations itself; more tokens quantize
into the workspace and run the decode GEMM.  Either way the float32 and bf16 outputs must equal
the two-launch path's bit for bit (same codes, scales, K split and summation order), and they are
held to the oracle's tolerance from the same bf16 inputs."""
import functools

import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, key, fmt, edge=False):
    x = workloads.activations(M, K, key=(3, 60, key, M))
    if edge:
        xf = workloads.bf16_bits_to_f32(x)
        xf[0, :128] = 0.0                                 # a zero group: scale 0, codes +-0
        if M > 1:
            xf[1, 128:256] *= np.float32(2.0 ** -118)     # a subnormal scale: IEEE quotient path
        x = workloads.f32_to_bf16_bits(xf)
    wq, sw = _weights(N, K, key, fmt)
    return x, wq, sw


@functools.lru_cache(maxsize=None)
def _weights(N, K, key, fmt):
    return blockquant.weight_quant(workloads.weights(N, K, key=(3, 61, key, N)), fmt)


def _oracle(x, wq, sw, fmt):
    aq, sa = blockquant.act_quant(x)
    return gemm.gemm_ref(aq, sa, wq, sw, fmt)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64])
@pytest.mark.parametrize("N,K", [(512, 2048), (1024, 4096), (4096, 4608), (4096, 4096), (12288, 1536)])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_fused_matches_two_launch_path_and_oracle(dev, M, N, K, fmt):
    x, wq, sw = _inputs(M, N, K, key=N + K, fmt=fmt, edge=True)
    xd = to_dev_bf16(x, dev)
    wqd, swd = torch.from_numpy(wq).to(dev), torch.from_numpy(sw).to(dev)
    one_launch = (M <= 4 and K >= 4096) or (M <= 8 and N * K <= (16 << 20))
    assert (fgb.gemm_fused_quant_workspace_bytes(M, N, K) == 0) == one_launch
    y32 = fgb.gemm_fused_quant(xd, wqd, swd, out_dtype=torch.float32)
    q, sa = fgb.quantize(xd)
    y32_two = fgb.gemm(q, sa, wqd, swd, out_dtype=torch.float32)
    y16 = fgb.gemm_fused_quant(xd, wqd, swd, out_dtype=torch.bfloat16)
    y16_two = fgb.gemm(q, sa, wqd, swd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), y32_two.view(torch.int32))
    assert torch.equal(y16.view(torch.int16), y16_two.view(torch.int16))
    yref = _oracle(x, wq, sw, fmt)
    y32n = y32.cpu().numpy()
    check_t1(y32n, yref)
    check_t2(bf16_tensor_to_f64(y16), yref)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32n.astype(np.float64)))


def test_fused_strided_input_and_output(dev):
    M, N, K = 12, 1024, 2048
    x, wq, sw = _inputs(M, N, K, key=7, fmt="f32")
    buf = torch.zeros((M, K + 128), dtype=torch.bfloat16, device=dev)
    buf[:, :K] = to_dev_bf16(x, dev)
    out = torch.full((M, N + 64), -7.0, dtype=torch.float32, device=dev)
    fgb.gemm_fused_quant(buf[:, :K], torch.from_numpy(wq).to(dev), torch.from_numpy(sw).to(dev),
                         out=out[:, :N])
    o = out.cpu().numpy()
    assert np.all(o[:, N:] == -7.0)
    check_t1(o[:, :N], _oracle(x, wq, sw, "f32"))


def test_fused_rejects_large_m(dev):
    x = torch.zeros((65, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        fgb.gemm_fused_quant(x, torch.zeros((256, 256), dtype=torch.uint8, device=dev),
                             torch.ones((2, 2), dtype=torch.float32, device=dev))
