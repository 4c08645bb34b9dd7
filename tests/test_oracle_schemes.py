"""Pins for the oracle's other scaling schemes (CPU): E5M2 codes, per-token / per-channel
quantization (FP8_DYNAMIC), static per-tensor quantization, and the GEMM under those scales.

Kinds of pin: an exact-rational restatement of the definition (float32 rounding on Fractions,
nearest-code search over the format's table), the format's printed maximum reached by the
largest element, reductions to the already pinned block functions (one group spanning a row,
block scales that are constant per row or per 128 rows), an exact-integer GEMM checked with
Python integers, and one dot product in exact rationals.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import blockquant, fp8, gemm, schemes
from tests.test_oracle_quant import rn32

_E5M2_POS = [(c, Fraction(float(v))) for c, v in zip(range(0x7C), fp8.dec_e5m2(np.arange(0x7C)))]
_E4M3_POS = [(c, Fraction(float(v))) for c, v in zip(range(0x7F), fp8.dec_e4m3(np.arange(0x7F)))]
_TABLE = {"e4m3": (_E4M3_POS, 448, 0x7E), "e5m2": (_E5M2_POS, 57344, 0x7B)}


def table_round(r: Fraction, negative: bool, code: str) -> int:
    """Nearest finite code by search (ties to the even code), saturating at the maximum."""
    pos, mx, top = _TABLE[code]
    a = abs(r)
    if a >= mx:
        c = top
    else:
        best = min(abs(a - v) for _, v in pos)
        cands = [c for c, v in pos if abs(a - v) == best]
        c = ([k for k in cands if k % 2 == 0] or cands)[0]
    return c | (0x80 if negative else 0)


def rational_quant(xs, code, s=None):
    """Codes (and the scale, if not given) of one group by the definition, exactly."""
    fx = [Fraction(float(v)) for v in xs]
    if s is None:
        s = rn32(max(abs(v) for v in fx) / _TABLE[code][1])
    else:
        s = Fraction(float(np.float32(s)))
    out = []
    for v, raw in zip(fx, xs):
        neg = math.copysign(1.0, float(raw)) < 0
        out.append((0x80 if neg else 0) if s == 0 else table_round(rn32(v / s), neg, code))
    return out, s


def _rows(M, K, key):
    return workloads.bf16_bits_to_f32(workloads.activations(M, K, key=key))


# ------------------------------------------------------------------------------------------
# E5M2 codes in the group quantizer
# ------------------------------------------------------------------------------------------
def test_e5m2_group_quant_rational_definition():
    x = _rows(3, 256, (1, 30, 0, 0))
    x[0, :128] *= np.float32(1e-30)   # tiny group (subnormal E5M2 codes)
    x[1, 128:] = 0.0                  # zero group
    q, s = blockquant.act_quant(x, code="e5m2")
    for m in range(3):
        for g in range(2):
            codes, sg = rational_quant(x[m, 128 * g:128 * (g + 1)], "e5m2")
            assert Fraction(float(s[m, g])) == sg
            assert q[m, 128 * g:128 * (g + 1)].tolist() == codes, (m, g)


def test_e5m2_max_element_reaches_57344():
    x = workloads.activations(32, 1024, key=(1, 31, 0, 0))
    q, s = blockquant.act_quant(x, code="e5m2")
    xf = workloads.bf16_bits_to_f32(x).reshape(32, 8, 128)
    idx = np.argmax(np.abs(xf), axis=2)
    top = np.take_along_axis(q.reshape(32, 8, 128), idx[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7B)   # +-57344, the printed E5M2 maximum


def test_e5m2_weight_blocks_and_qdq_bound():
    w = workloads.weights(256, 384, key=(1, 32, 1, 0))
    q, s = blockquant.weight_quant(w, "f32", code="e5m2")
    wf = workloads.bf16_bits_to_f32(w).astype(np.float64)
    sx = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
    d = fp8.dec_e5m2(q)
    a = np.abs(d)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -14)
    half_ulp = 0.5 * 2.0 ** (e - 2)
    r = wf / sx
    assert np.all(np.abs(d - r) <= half_ulp + 2.0 ** -23 * np.abs(r))
    for nb in range(2):
        for kb in range(3):
            blk = wf[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)]
            assert Fraction(float(s[nb, kb])) == rn32(Fraction(float(np.max(np.abs(blk)))) / 57344)
    with pytest.raises(ValueError):
        blockquant.weight_quant(w, "ue8m0", code="e5m2")


# ------------------------------------------------------------------------------------------
# per-token / per-channel (FP8_DYNAMIC)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("code", ["e4m3", "e5m2"])
def test_token_quant_rational_definition(code):
    x = _rows(4, 384, (1, 33, 0, 0))
    x[2] = 0.0
    x[3] *= np.float32(2.0 ** -100)
    q, s = schemes.token_quant(x, code)
    assert s.shape == (4,)
    for m in range(4):
        codes, sm = rational_quant(x[m], code)
        assert Fraction(float(s[m])) == sm
        assert q[m].tolist() == codes, m


def test_token_quant_reduces_to_group_quant_at_k128():
    x = workloads.activations(16, 128, key=(1, 34, 0, 0))
    q, s = schemes.token_quant(x)
    qg, sg = blockquant.act_quant(x)
    assert np.array_equal(q, qg) and np.array_equal(s.view(np.uint32), sg[:, 0].view(np.uint32))


def test_token_quant_invariants():
    x = _rows(6, 512, (1, 35, 0, 0))
    q, s = schemes.token_quant(x)
    # the row's largest element takes the maximum code
    idx = np.argmax(np.abs(x), axis=1)
    assert np.all((q[np.arange(6), idx] & 0x7F) == 0x7E)
    # a column permutation permutes the codes and keeps the scale
    perm = np.random.default_rng(1).permutation(512)
    q2, s2 = schemes.token_quant(x[:, perm])
    assert np.array_equal(q2, q[:, perm]) and np.array_equal(s2, s)
    # scaling a row by a power of two scales its scale and keeps its codes
    q3, s3 = schemes.token_quant((x * np.float32(2.0 ** 9)).astype(np.float32))
    assert np.array_equal(q3, q) and np.array_equal(s3, (s * np.float32(2.0 ** 9)).astype(np.float32))
    # rows are independent
    q4, s4 = schemes.token_quant(x[::-1].copy())
    assert np.array_equal(q4, q[::-1]) and np.array_equal(s4, s[::-1])


def test_channel_weight_quant_is_per_output_row():
    w = workloads.weights(8, 256, key=(1, 36, 1, 0))
    q, s = schemes.channel_weight_quant(w)
    wf = workloads.bf16_bits_to_f32(w)
    for n in range(8):
        codes, sn = rational_quant(wf[n], "e4m3")
        assert Fraction(float(s[n])) == sn and q[n].tolist() == codes


# ------------------------------------------------------------------------------------------
# static per-tensor quantization
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("code", ["e4m3", "e5m2"])
def test_static_quant_rational_definition_and_saturation(code):
    x = _rows(2, 256, (1, 37, 0, 0))
    s = np.float32(0.013 if code == "e4m3" else 1e-4)   # small: the outliers saturate
    q = schemes.static_quant(x, s, code)
    for m in range(2):
        codes, _ = rational_quant(x[m], code, s=s)
        assert q[m].tolist() == codes
    big = np.abs(x) > np.float64(_TABLE[code][1]) * float(s)
    assert big.any() and np.all((q[big] & 0x7F) == _TABLE[code][2])


def test_static_quant_divides_by_the_scale():
    """Division by the given scale, not multiplication by its reciprocal: for this pair (found by
    a search over random scales) fl32(x / s) and fl32(x * fl32(1 / s)) straddle an E4M3 rounding
    point; the rational definition gives code 0x10."""
    s = np.array([0x3F3BDEF8], dtype=np.uint32).view(np.float32)[0]
    x = np.array([[0x3CB6]], dtype=np.uint16)
    codes, _ = rational_quant(workloads.bf16_bits_to_f32(x)[0], "e4m3", s=s)
    assert codes == [0x10]
    assert schemes.static_quant(x, s).tolist() == [[0x10]]


def test_static_quant_with_the_dynamic_scale_reduces_to_group_quant():
    x = workloads.activations(1, 128, key=(1, 38, 0, 0))
    qg, sg = blockquant.act_quant(x)
    assert np.array_equal(schemes.static_quant(x, sg[0, 0]), qg)
    with pytest.raises(ValueError):
        schemes.static_quant(x, 0.0)


# ------------------------------------------------------------------------------------------
# GEMM under per-token/per-channel and static scales
# ------------------------------------------------------------------------------------------
def test_token_channel_gemm_reduces_to_block_gemm():
    """Per-channel scales that are constant over each 128 rows and per-token scales are a
    special case of the (pinned) block GEMM."""
    M, N, K = 20, 256, 384
    rng = np.random.default_rng(5)
    aq, _ = blockquant.act_quant(workloads.activations(M, K, key=(1, 39, 0, 0)))
    wq, _ = blockquant.weight_quant(workloads.weights(N, K, key=(1, 39, 1, 0)))
    sa = rng.uniform(0.001, 0.01, size=M).astype(np.float32)
    sw_blocks = rng.uniform(0.0001, 0.001, size=N // 128).astype(np.float32)
    sw = np.repeat(sw_blocks, 128)
    y = schemes.scaled_gemm_ref(aq, sa, wq, sw, act="token", weight="channel")
    yb = gemm.gemm_ref(aq, np.repeat(sa[:, None], K // 128, axis=1), wq,
                       np.repeat(sw_blocks[:, None], K // 128, axis=1))
    assert np.max(np.abs(y - yb)) <= 1e-12 * np.max(np.abs(yb))


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_tensor_block_gemm_reduces_to_block_gemm(fmt):
    M, N, K = 9, 256, 512
    aq, _ = blockquant.act_quant(workloads.activations(M, K, key=(1, 40, 0, 0)))
    wq, sw = blockquant.weight_quant(workloads.weights(N, K, key=(1, 40, 1, 0)), fmt)
    s_act = np.float32(0.0123)
    y = schemes.scaled_gemm_ref(aq, s_act, wq, sw, act="tensor", weight="block", w_scale_fmt=fmt)
    yb = gemm.gemm_ref(aq, np.full((M, K // 128), s_act, dtype=np.float32), wq, sw, fmt)
    assert np.max(np.abs(y - yb)) <= 1e-12 * np.max(np.abs(yb))


@pytest.mark.parametrize("codes", [("e5m2", "e5m2"), ("e4m3", "e4m3"), ("e4m3", "e5m2")])
def test_exact_integer_gemm_with_python_ints(codes):
    """Codes that decode to small integers, unit scales: y is an exact integer, checked against
    Python integer arithmetic."""
    a_code, w_code = codes
    rng = np.random.default_rng(6)
    ints = np.array([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], dtype=np.float32)
    A = rng.choice(ints, size=(5, 256))
    W = rng.choice(ints, size=(7, 256))
    aq = blockquant.encode(A, a_code)
    wq = blockquant.encode(W, w_code)
    y = schemes.scaled_gemm_ref(aq, np.ones(5, np.float32), wq, np.ones(7, np.float32), act="token",
                                weight="channel", a_code=a_code, w_code=w_code)
    exact = [[sum(int(a) * int(b) for a, b in zip(A[m], W[n])) for n in range(7)] for m in range(5)]
    assert y.tolist() == exact


def test_e5m2_dot_product_in_rationals():
    rng = np.random.default_rng(7)
    finite = [c for c in range(256) if (c & 0x7F) < 0x7C]
    a = rng.choice(finite, size=(1, 128)).astype(np.uint8)
    w = rng.choice(finite, size=(1, 128)).astype(np.uint8)
    y = schemes.scaled_gemm_ref(a, np.float32(0.5), w, np.float32([3.0]), act="tensor", weight="channel",
                                a_code="e5m2", w_code="e5m2")
    terms = [Fraction(float(fp8.dec_e5m2(i))) * Fraction(float(fp8.dec_e5m2(j))) for i, j in zip(a[0], w[0])]
    exact = sum(terms) * Fraction(3, 2)
    # every product is exact in float64; only the float64 additions may round
    bound = 130 * 2.0 ** -53 * float(sum(abs(t) for t in terms)) * 1.5
    assert abs(Fraction(float(y[0, 0])) - exact) <= Fraction(bound)
    assert abs(exact) > 1000 * Fraction(bound)   # the check is not vacuous
