"""Pins for the oracle's block-scaled GEMM, grouped GEMM and bf16 rounding (CPU).

Independent checks: a dense float64 brute force written element by element from the decoded
operands; an exact-integer special case computed with Python integers; exact homogeneity in
the weight scales; a single 128-long dot product in exact rational arithmetic; reduction of
the grouped GEMM to the dense one; bf16 rounding against an exhaustive table search.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import blockquant, fp8, gemm


def _tiny(M=64, N=256, K=384, key=0, fmt="f32"):
    x = workloads.activations(M, K, key=(key, 0, 0, 0))
    w = workloads.weights(N, K, key=(key, 0, 1, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = blockquant.weight_quant(w, fmt)
    return aq, sa, wq, sw


def _dense_bruteforce(aq, sa, wq, sw, fmt):
    """Dequantize every element with its own scale, then a plain float64 matmul."""
    M, K = aq.shape
    N = wq.shape[0]
    swv = np.asarray(sw, np.float32).astype(np.float64) if fmt == "f32" else fp8.dec_ue8m0(sw)
    A = np.empty((M, K))
    W = np.empty((N, K))
    da, dw = fp8.dec_e4m3(aq), fp8.dec_e4m3(wq)
    for k in range(K):
        A[:, k] = da[:, k] * sa[:, k // 128]
        W[:, k] = dw[:, k] * swv[np.arange(N) // 128, k // 128]
    return A @ W.T


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_blockwise_equals_dense_bruteforce(fmt):
    aq, sa, wq, sw = _tiny(fmt=fmt)
    y = gemm.gemm_ref(aq, sa, wq, sw, fmt)
    yd = _dense_bruteforce(aq, sa, wq, sw, fmt)
    assert np.max(np.abs(y - yd)) <= 1e-12 * np.max(np.abs(yd))
    yf = gemm.gemm_ref_fast(aq, sa, wq, sw, fmt)
    assert np.max(np.abs(y - yf)) <= 1e-12 * np.max(np.abs(yd))


def test_exact_integer_special_case():
    """Every group/block holds +-448, so all scales are exactly 1; other entries are small
    E4M3 integers; y is then an exact integer computed here with Python ints."""
    rng = np.random.default_rng(3)
    M, N, K = 48, 256, 512
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
    A = rng.choice(ints, size=(M, K))
    W = rng.choice(ints, size=(N, K))
    A[:, ::128] = 448.0
    W[:, ::128] = -448.0
    W[::128, 1::128] = 448.0
    aq, sa = blockquant.act_quant(A)
    wq, sw = blockquant.weight_quant(W, "f32")
    assert np.all(sa == 1.0) and np.all(sw == 1.0)
    y = gemm.gemm_ref(aq, sa, wq, sw)
    Ai = A.astype(np.int64)
    Wi = W.astype(np.int64)
    yi = Ai @ Wi.T  # exact integer product (int64, |y| < 2^31 here)
    assert np.array_equal(y, yi.astype(np.float64))


def test_homogeneity_in_weight_scales():
    aq, sa, wq, sw = _tiny(M=16, N=128, K=256, key=1)
    y = gemm.gemm_ref(aq, sa, wq, sw)
    y2 = gemm.gemm_ref(aq, sa, wq, (sw * np.float32(2)).astype(np.float32))
    assert np.array_equal(y2, 2 * y)


def test_single_dot_product_exact():
    aq, sa, wq, sw = _tiny(M=1, N=128, K=128, key=2)
    y = gemm.gemm_ref(aq, sa, wq, sw)
    for n in [0, 5, 77, 127]:
        acc = Fraction(0)
        for k in range(128):
            acc += Fraction(float(fp8.dec_e4m3(aq[0, k]))) * Fraction(float(fp8.dec_e4m3(wq[n, k])))
        exp = float(acc * Fraction(float(sa[0, 0])) * Fraction(float(sw[0, 0])))
        assert abs(y[0, n] - exp) <= 1e-15 * abs(exp) + 1e-300


def test_partial_sums_are_exact_multiples():
    """Every per-block partial is j * 2^-18 with |j| < 2^53 (so float64 sums exactly)."""
    aq, sa, wq, sw = _tiny(M=8, N=128, K=128, key=4)
    P = fp8.dec_e4m3(aq) @ fp8.dec_e4m3(wq).T
    j = P * 2.0 ** 18
    assert np.array_equal(j, np.round(j)) and np.all(np.abs(j) < 2.0 ** 53)


def test_grouped_reduces_to_dense_and_handles_empty_experts():
    rng = np.random.default_rng(5)
    E, N, K = 4, 128, 256
    counts = [7, 0, 33, 24]
    offsets = workloads.offsets_from_counts(counts)
    T = offsets[-1]
    x = workloads.activations(T, K, key=(0, 8, 0, 0))
    aq, sa = blockquant.act_quant(x)
    wq = np.empty((E, N, K), np.uint8)
    sw = np.empty((E, 1, 2), np.float32)
    for e in range(E):
        wq[e], sw[e] = blockquant.weight_quant(workloads.weights(N, K, key=(0, 8, 1, e)))
    y = gemm.grouped_ref(aq, sa, wq, sw, offsets)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            assert np.array_equal(y[r0:r1], gemm.gemm_ref(aq[r0:r1], sa[r0:r1], wq[e], sw[e]))
    # E = 1 is the dense GEMM; all rows in one expert
    y1 = gemm.grouped_ref(aq, sa, wq[2:3], sw[2:3], np.array([0, T]))
    assert np.array_equal(y1, gemm.gemm_ref(aq, sa, wq[2], sw[2]))
    y0 = gemm.grouped_ref(aq, sa, wq, sw, np.array([0, 0, T, T, T]))
    assert np.array_equal(y0, gemm.gemm_ref(aq, sa, wq[1], sw[1]))
    with pytest.raises(ValueError):
        gemm.grouped_ref(aq, sa, wq, sw, np.array([0, 5, 3, T, T]))


def _bf16_table():
    bits = np.arange(0, 0x7F81, dtype=np.uint32)  # +0 .. +inf
    return bits, (bits << 16).view(np.float32).astype(np.float64)


def test_bf16_rne_bruteforce():
    bits, vals = _bf16_table()
    rng = np.random.default_rng(6)
    fin = vals[np.isfinite(vals)]
    mids = (fin[:-1] + fin[1:]) / 2
    probes = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                             mids[::97], np.nextafter(mids[::97], 0), np.nextafter(mids[::97], np.inf)])
    got = gemm.bf16_rne(probes)
    a = np.abs(probes)
    idx = np.searchsorted(fin, a)
    lo = fin[np.clip(idx - 1, 0, fin.size - 1)]
    hi = fin[np.clip(idx, 0, fin.size - 1)]
    lo_bits = np.clip(idx - 1, 0, fin.size - 1)
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (lo_bits % 2 == 1))
    exp = np.where(a == hi, hi, np.where(pick_hi, hi, lo))
    exp = np.copysign(exp, probes)
    assert np.array_equal(got, exp)


def test_bf16_rne_matches_torch_on_float32_values():
    x = np.random.default_rng(7).standard_normal(100000).astype(np.float32) * np.float32(1e3)
    t = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(gemm.bf16_rne(x.astype(np.float64)), t)


def test_batched_reduces_to_grouped_with_empty_and_full_experts():
    """The masked batched layout equals the contiguous grouped layout on the valid rows: gather
    them in expert order, offsets from the running sum of the counts (zero-count experts, full
    slots and a partly filled slot included)."""
    E, max_m, N, K = 5, 24, 256, 384
    counts = np.array([0, 24, 7, 0, 1])
    rng = np.random.default_rng(11)
    aq, sa = blockquant.act_quant(workloads.activations(E * max_m, K, key=(0, 70, 0, 0)))
    wq = np.stack([blockquant.weight_quant(workloads.weights(N, K, key=(0, 70, 1, e)))[0] for e in range(E)])
    sw = rng.uniform(1e-4, 1e-3, size=(E, N // 128, K // 128)).astype(np.float32)
    y, valid = gemm.batched_ref(aq, sa, wq, sw, counts, max_m)
    rows = np.concatenate([np.arange(e * max_m, e * max_m + counts[e]) for e in range(E)])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    yg = gemm.grouped_ref(aq[rows], sa[rows], wq, sw, offsets)
    assert valid.sum() == counts.sum() and np.array_equal(np.nonzero(valid)[0], rows)
    assert np.array_equal(y[rows], yg)
    assert np.all(y[~valid] == 0)
    with pytest.raises(ValueError):
        gemm.batched_ref(aq, sa, wq, sw, np.array([0, 25, 0, 0, 0]), max_m)

