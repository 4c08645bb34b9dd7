"""GPU parity: act_quant_group128 and weight_quant_block128 bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant

pytestmark = pytest.mark.gpu


def _to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)


def _run_quant(bits, dev, ld=None):
    M, K = bits.shape
    x = _to_dev_bf16(bits, dev)
    if ld is not None and ld > K:  # strided input: a wider buffer, use the first K columns
        buf = torch.zeros((M, ld), dtype=torch.bfloat16, device=dev)
        buf[:, :K] = x
        x = buf[:, :K]
    q, s_a = fgb.quantize(x)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s_a[:, :M].t().contiguous().cpu().numpy()


def _check(bits, dev, ld=None):
    q, s = _run_quant(bits, dev, ld)
    qe, se = blockquant.act_quant(bits)
    assert np.array_equal(s.view(np.uint32), se.view(np.uint32)), "scales differ"
    bad = np.argwhere(q != qe)
    assert bad.size == 0, (bad[:5], q[tuple(bad[0])], qe[tuple(bad[0])])


def test_tiny_config(dev):
    _check(workloads.activations(64, 1024, key=(0, 0, 0, 0)), dev)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (17, 384), (255, 1024), (1000, 4096), (4097, 128)])
def test_ragged_shapes(dev, M, K):
    _check(workloads.activations(M, K, key=(0, 1, 0, M)), dev)


def test_strided_input(dev):
    _check(workloads.activations(33, 512, key=(0, 2, 0, 0)), dev, ld=640)


def test_edge_groups(dev):
    x = workloads.bf16_bits_to_f32(workloads.activations(8, 1024, key=(0, 3, 0, 0)))
    x[0, 0:128] = 0.0                                     # amax 0: scale 0, codes +0
    x[0, 128:256] = -0.0                                  # codes -0
    x[1, 0:128] *= np.float32(2.0 ** -125)                # tiny amax: subnormal scale
    x[1, 128:256] = np.float32(2.0 ** -133) * np.arange(128, dtype=np.float32)  # bf16 subnormals
    x[2, 0:128] = np.float32(3.0e38) * np.sign(x[2, 0:128])  # near bf16 max
    x[2, 128:256] = np.float32(448.0)                     # exact scale 1
    x[3, 0:128] = np.float32(1.0)
    x[3, 5] = np.float32(-896.0)                          # exact scale 2, negative max
    x[4, :] = np.float32(2.0 ** -100) * x[4, :]
    x[5, 0:128] = np.float32(1e-30)
    bits = workloads.f32_to_bf16_bits(x)
    _check(bits, dev)


def test_all_bf16_magnitudes_against_a_set_of_maxima(dev):
    """Every finite bf16 value x with |x| <= amax, for 48 group maxima spread over the range;
    each group is [amax, x_1 .. x_127]."""
    allb = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    vals = workloads.bf16_bits_to_f32(allb)
    rng = np.random.default_rng(4)
    amax_bits = np.unique(np.concatenate([
        np.array([0x3F80, 0x43E0, 0x4000, 0x3C00, 0x4780, 0x0080, 0x0F00, 0x7F7F], dtype=np.uint16),
        rng.integers(0x0100, 0x7F7F, 40).astype(np.uint16)]))
    rows = []
    for ab in amax_bits:
        a = workloads.bf16_bits_to_f32(np.array([ab], np.uint16))[0]
        xs = allb[vals <= a]
        xs = np.concatenate([xs, xs | np.uint16(0x8000)])
        pad = (-len(xs)) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        grp = np.concatenate([np.full((xs.shape[0], 1), ab, np.uint16), xs], axis=1)
        rows.append(grp)
    g = np.concatenate(rows)
    g = g[: (g.shape[0] // 8) * 8].reshape(-1, 8 * 128)  # 8 groups per row, K = 1024
    _check(g, dev)


@pytest.mark.parametrize("M,K", [(4096, 4096), (4096, 14336), (8192, 1536), (8192, 18432), (32768, 7168), (32768, 2048)])
def test_config_shapes_sampled_rows(dev, M, K):
    """Full-size activation quantization as the GEMM inputs use it; 96 sampled rows checked."""
    bits = workloads.activations(M, K, key=(0, 10, 0, K))
    q, s = _run_quant(bits, dev)
    rows = np.random.default_rng(M + K).choice(M, 96, replace=False)
    qe, se = blockquant.act_quant(bits[rows])
    assert np.array_equal(s[rows].view(np.uint32), se.view(np.uint32))
    assert np.array_equal(q[rows], qe)


@pytest.mark.parametrize("fmt", ["float", "ue8m0"])
def test_weight_quant(dev, fmt):
    w = workloads.weights(512, 1024, key=(0, 11, 1, 0))
    wf = workloads.bf16_bits_to_f32(w)
    wf[0:128, 0:128] = 0.0                      # zero block
    wf[128:256, 128:256] *= np.float32(1e-30)   # tiny block
    w = workloads.f32_to_bf16_bits(wf)
    q, s = fgb.quantize_weight(_to_dev_bf16(w, dev), fmt)
    torch.cuda.synchronize()
    qe, se = blockquant.weight_quant(w, "f32" if fmt == "float" else "ue8m0")
    s_np = s.cpu().numpy()
    if fmt == "ue8m0":
        assert np.array_equal(s_np, se)
    else:
        assert np.array_equal(s_np.view(np.uint32), se.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qe)


def test_fast_quotient_selftest(dev):
    """The quantizers' reciprocal-and-correct quotient gives the IEEE quotient's E4M3 code for
    every positive finite bf16 amax and every bf16 |x| <= amax, both signs (~1.07e9 pairs)."""
    code_bad, quot_bad, quot_bad_big = fgb.selftest_quotients()
    assert code_bad == 0
    # the last-bit differences come only from residuals below the float32 normal range, i.e.
    # tiny quotients, which encode as +-0 whichever way they round
    assert quot_bad_big == 0
    print(f"float32 quotient mismatches (codes equal, all below 2^-13): {quot_bad}")
