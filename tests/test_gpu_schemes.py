"""GPU parity for the other FP8 schemes, through the C-ABI, against the oracle (oracle/schemes.py):
per-token and per-channel quantization (FP8_DYNAMIC), quantization with a given per-tensor scale
(static activations), E5M2 codes, and the GEMM under those scales.

Quantization: codes and scales bit-exact.  GEMM: float32 mode max|y - y_ref| <= 2e-3 max|y_ref|,
bf16 mode per element |y - y_ref| <= 2e-3 max|y_ref| + 1 bf16 ulp, bf16 == RNE(float32), and an
exact-integer case bit for bit.  Shapes cover the decode kernel at 8, 16, 32 and 64 staged rows
(M = 1, 8, 9, 17, 33, 64) and both prefill tilings (N a multiple of 256 with K >= 1024, and not).
"""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm, schemes
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, to_dev_bf16

pytestmark = pytest.mark.gpu

CODES = ["e4m3", "e5m2"]


def _x(M, K, key):
    return workloads.activations(M, K, key=(2, 50, key, M * 7 + K))


def _w(N, K, key):
    return workloads.weights(N, K, key=(2, 51, key, N * 7 + K))


def _f32_bits(t):
    return t.cpu().numpy().view(np.uint32)


# ------------------------------------------------------------------------------------------
# quantizers
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("M,K", [(1, 128), (7, 1024), (33, 4096), (130, 7168)])
def test_per_token_quant_bit_exact(dev, code, M, K):
    x = _x(M, K, 1)
    xf = workloads.bf16_bits_to_f32(x)
    if M > 2:
        xf[1] = 0.0                               # a zero row: scale 0, codes +-0
        xf[2] *= np.float32(2.0 ** -110)          # a tiny row: subnormal scale
    x = workloads.f32_to_bf16_bits(xf)
    q, s = fgb.quantize_per_token(to_dev_bf16(x, dev), code)
    torch.cuda.synchronize()
    qe, se = schemes.token_quant(x, code)
    assert np.array_equal(_f32_bits(s), se.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qe)


def test_per_token_quant_strided_input(dev):
    M, K = 20, 512
    x = _x(M, K, 2)
    buf = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=dev)
    buf[:, :K] = to_dev_bf16(x, dev)
    q, s = fgb.quantize_per_token(buf[:, :K])
    qe, se = schemes.token_quant(x)
    assert np.array_equal(q.cpu().numpy(), qe) and np.array_equal(_f32_bits(s), se.view(np.uint32))


@pytest.mark.parametrize("code", CODES)
def test_per_channel_weight_quant_bit_exact(dev, code):
    w = _w(384, 2048, 3)
    q, s = fgb.quantize_weight_per_channel(to_dev_bf16(w, dev), code)
    qe, se = schemes.channel_weight_quant(w, code)
    assert np.array_equal(_f32_bits(s), se.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qe)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("scale", [0.013, 1e-4, 3.5, 0.7338709831237793])
def test_static_quant_bit_exact(dev, code, scale):
    x = _x(37, 1024, 4)
    s = np.float32(scale)
    q = fgb.quantize_static(to_dev_bf16(x, dev), torch.tensor([s], dtype=torch.float32, device=dev), code)
    assert np.array_equal(q.cpu().numpy(), schemes.static_quant(x, s, code))


def test_static_quant_division_golden_pair(dev):
    """The pair on which dividing by the scale and multiplying by its reciprocal differ."""
    s = np.array([0x3F3BDEF8], dtype=np.uint32).view(np.float32)
    x = np.full((1, 128), 0x3CB6, dtype=np.uint16)
    q = fgb.quantize_static(to_dev_bf16(x, dev), torch.from_numpy(s).to(dev))
    assert np.all(q.cpu().numpy() == 0x10)


@pytest.mark.parametrize("code", CODES)
def test_quantizers_streamed_size_bit_exact(dev, code):
    """Inputs of 16 MiB or more take the kernels' streamed form (non-temporal loads and stores):
    per-token and static codes, and per-token scales, on sampled rows incl. the first and last."""
    M, K = 2048, 4096  # 16 MiB of bf16
    x = _x(M, K, 31)
    xd = to_dev_bf16(x, dev)
    q, s = fgb.quantize_per_token(xd, code)
    st = np.float32(0.0123)
    qs = fgb.quantize_static(xd, torch.tensor([st], dtype=torch.float32, device=dev), code)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(31).choice(M, 40, replace=False)]))
    qe, se = schemes.token_quant(x[rows], code)
    assert np.array_equal(q.cpu().numpy()[rows], qe)
    assert np.array_equal(_f32_bits(s)[rows], se.view(np.uint32))
    assert np.array_equal(qs.cpu().numpy()[rows], schemes.static_quant(x[rows], st, code))


def test_e5m2_block_weight_quant_bit_exact(dev):
    w = _w(256, 1024, 5)
    wf = workloads.bf16_bits_to_f32(w)
    wf[:128, :128] = 0.0
    wf[128:, 128:256] *= np.float32(1e-30)
    w = workloads.f32_to_bf16_bits(wf)
    q, s = fgb.quantize_weight(to_dev_bf16(w, dev), "float", code="e5m2")
    qe, se = blockquant.weight_quant(w, "f32", code="e5m2")
    assert np.array_equal(_f32_bits(s), se.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qe)


# ------------------------------------------------------------------------------------------
# GEMM
# ------------------------------------------------------------------------------------------
def _operands(M, N, K, act, weight, code, fmt="f32", key=0):
    x, w = _x(M, K, 10 + key), _w(N, K, 10 + key)
    if act == "token":
        aq, sa = schemes.token_quant(x, code)
    else:
        sa = np.float32(0.05 if code == "e4m3" else 4e-4)
        aq = schemes.static_quant(x, sa, code)
    if weight == "channel":
        wq, sw = schemes.channel_weight_quant(w, code)
    else:
        wq, sw = blockquant.weight_quant(w, fmt, code=code)
    return aq, sa, wq, sw


def _run(ops, dev, act, code, out_dtype):
    aq, sa, wq, sw = ops
    sa_d = torch.from_numpy(np.atleast_1d(np.asarray(sa, dtype=np.float32)).copy()).to(dev)
    y = fgb.scaled_gemm(torch.from_numpy(aq).to(dev), sa_d, torch.from_numpy(wq).to(dev),
                        torch.from_numpy(np.ascontiguousarray(sw)).to(dev), act_scale=act, code=code,
                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


SHAPES = [(1, 256, 1024), (8, 384, 512), (9, 256, 2048), (17, 512, 1024), (33, 256, 1536), (64, 1024, 1024),
          (65, 256, 1024), (300, 384, 1024), (300, 512, 2048)]


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("act,weight", [("token", "channel"), ("tensor", "block"), ("tensor", "channel"),
                                        ("token", "block")])
def test_scaled_gemm_parity(dev, code, act, weight):
    for i, (M, N, K) in enumerate(SHAPES):
        ops = _operands(M, N, K, act, weight, code, key=i)
        yref = schemes.scaled_gemm_ref(*ops, act=act, weight=weight, a_code=code, w_code=code)
        y32 = _run(ops, dev, act, code, torch.float32).cpu().numpy()
        check_t1(y32, yref)
        y16 = _run(ops, dev, act, code, torch.bfloat16)
        check_t2(bf16_tensor_to_f64(y16), yref)
        assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64))), (M, N, K)


# decode shapes that reach each decode kernel: M <= 16 with >= 48 MiB of weights and K >= 8192
# (LDS-ring kernel); 16 < M <= 64 with more than 16 MiB of weights: the shared-ring kernel in one
# K slice (>= 160 weight blocks of 128 rows) or in several, with partials and the scaling
# reduction (fewer blocks)
DECODE_PATHS = [(4, 2048, 24576), (16, 2048, 24576), (17, 20480, 1024), (33, 20480, 1024), (64, 20480, 1024),
                (40, 4096, 8192), (64, 4096, 14336), (24, 4096, 4608), (32, 10240, 5248)]


@pytest.mark.parametrize("M,N,K", DECODE_PATHS)
@pytest.mark.parametrize("act,weight,code,fmt", [("token", "channel", "e4m3", "f32"), ("tensor", "block", "e5m2", "f32"),
                                                 ("token", "block", "e4m3", "ue8m0")])
def test_scaled_gemm_decode_kernels(dev, M, N, K, act, weight, code, fmt):
    ops = _operands(M, N, K, act, weight, code, fmt=fmt, key=40 + M)
    yref = schemes.scaled_gemm_ref(*ops, act=act, weight=weight, a_code=code, w_code=code, w_scale_fmt=fmt)
    y32 = _run(ops, dev, act, code, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run(ops, dev, act, code, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))


@pytest.mark.parametrize("M", [8, 64, 300])
def test_static_block_gemm_ue8m0(dev, M):
    N, K = 512, 1024
    ops = _operands(M, N, K, "tensor", "block", "e4m3", fmt="ue8m0", key=20 + M)
    yref = schemes.scaled_gemm_ref(*ops, act="tensor", weight="block", w_scale_fmt="ue8m0")
    check_t1(_run(ops, dev, "tensor", "e4m3", torch.float32).cpu().numpy(), yref)
    check_t2(bf16_tensor_to_f64(_run(ops, dev, "tensor", "e4m3", torch.bfloat16)), yref)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("M", [5, 40, 200])
def test_scaled_gemm_exact_integer_case(dev, code, M):
    """Codes that decode to small integers and unit scales: the float32 result is exact."""
    rng = np.random.default_rng(M)
    N, K = 256, 1024
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
    aq = blockquant.encode(rng.choice(ints, size=(M, K)), code)
    wq = blockquant.encode(rng.choice(ints, size=(N, K)), code)
    ops = (aq, np.ones(M, np.float32), wq, np.ones(N, np.float32))
    yref = schemes.scaled_gemm_ref(*ops, act="token", weight="channel", a_code=code, w_code=code)
    assert np.all(np.abs(yref) < 2 ** 24)
    y32 = _run(ops, dev, "token", code, torch.float32).cpu().numpy()
    assert np.array_equal(y32.astype(np.float64), yref)


@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("M", [4, 48, 256])
def test_fp8_dynamic_end_to_end(dev, code, M):
    """GPU per-token and per-channel quantization, then the GEMM, from bf16 inputs, against the
    oracle run from the same inputs."""
    N, K = 512, 2048
    x, w = _x(M, K, 30), _w(N, K, 30)
    q, sa = fgb.quantize_per_token(to_dev_bf16(x, dev), code)
    wq, sw = fgb.quantize_weight_per_channel(to_dev_bf16(w, dev), code)
    y = fgb.scaled_gemm(q, sa, wq, sw, act_scale="token", code=code)
    torch.cuda.synchronize()
    aq_e, sa_e = schemes.token_quant(x, code)
    wq_e, sw_e = schemes.channel_weight_quant(w, code)
    yref = schemes.scaled_gemm_ref(aq_e, sa_e, wq_e, sw_e, act="token", weight="channel", a_code=code, w_code=code)
    check_t2(bf16_tensor_to_f64(y), yref)


def test_scaled_gemm_rejects_group_scales_and_mixed_ue8m0(dev):
    aq = torch.zeros((16, 256), dtype=torch.uint8, device=dev)
    wq = torch.zeros((256, 256), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        fgb.scaled_gemm(aq, torch.ones(16, device=dev), wq, torch.ones((2, 2), dtype=torch.uint8, device=dev),
                        code="e5m2")
    with pytest.raises(ValueError):
        fgb.scaled_gemm(aq, torch.ones(16, device=dev), wq, torch.ones(256, device=dev), act_scale="group")
