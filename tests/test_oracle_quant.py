"""Pins for the oracle's activation and weight quantization (CPU).

Independent checks: hand-worked golden groups; an exact-rational restatement of the definition
(float32 rounding done on Fractions, E4M3 rounding by table search); invariants that any
correct implementation satisfies (maximum element saturates to +-448, half-ulp Q-DQ bound,
power-of-two scaling, permutation and group independence); UE8M0 closed forms.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import blockquant, fp8

GOLD = os.path.join(os.path.dirname(__file__), "golden", "act_quant_handworked.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _group_row(values, K=128):
    row = np.zeros(K, dtype=np.float32)
    row[: len(values)] = np.float32(values)
    return row


# ------------------------------------------------------------------------------------------
# exact-rational restatement of the definition
# ------------------------------------------------------------------------------------------
def rn32(q: Fraction) -> Fraction:
    """Round a rational to the nearest float32 (ties to even), gradual underflow, no overflow."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


_E4M3_POS = [(c, Fraction(float(v))) for c, v in zip(range(0x7F), fp8.dec_e4m3(np.arange(0x7F)))]


def e4m3_table_round(r: Fraction, negative: bool) -> int:
    a = abs(r)
    if a >= 448:
        code = 0x7E
    else:
        best = min(abs(a - v) for _, v in _E4M3_POS)
        cands = [c for c, v in _E4M3_POS if abs(a - v) == best]
        even = [c for c in cands if c % 2 == 0]
        code = (even or cands)[0]
    return code | (0x80 if negative else 0)


def rational_group(xs):
    """Codes and scale of one group by the definition, in exact rational arithmetic."""
    fx = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fx)
    s = rn32(amax / 448)
    codes = []
    for v, raw in zip(fx, xs):
        neg = math.copysign(1.0, float(raw)) < 0
        if s == 0:
            codes.append(0x80 if neg else 0x00)
        else:
            codes.append(e4m3_table_round(rn32(v / s), neg))
    return s, codes


# ------------------------------------------------------------------------------------------
def test_golden_handworked_groups():
    g = _gold()
    rows = np.stack([_group_row(grp["x"]) for grp in g["groups"]])
    q, s = blockquant.act_quant(rows)
    for i, grp in enumerate(g["groups"]):
        assert s[i, 0] == np.float32(grp["scale"])
        exp = [int(c, 16) for c in grp["codes"]]
        assert q[i, : len(exp)].tolist() == exp, grp["why"]
        assert np.all(q[i, len(exp):] == 0)


def test_golden_ue8m0_scale_choice():
    u = _gold()["ue8m0"]
    assert fp8.ue8m0_from_amax(np.float32(u["amax"])).tolist() == u["codes"]


def test_division_by_stored_scale_reading():
    pairs = _gold()["division_reading"]["pairs"]
    rows = np.stack([_group_row([a, x]) for x, a in pairs])
    q, s = blockquant.act_quant(rows)
    for i, (x, a) in enumerate(pairs):
        s_exp, codes = rational_group([a, x])
        assert Fraction(float(s[i, 0])) == s_exp
        assert q[i, 1] == codes[1]
        # the multiply-by-reciprocal variant differs here (that is why the pair is listed)
        alt = fp8.enc_e4m3_sat(np.float32(x) * (np.float32(448.0) / np.float32(a)))
        assert alt != codes[1]


def test_rational_definition_on_recipe_rows():
    x = workloads.activations(6, 512, key=(0, 99, 0, 0))
    x = workloads.bf16_bits_to_f32(x)
    # add special groups: tiny amax (subnormal scale), bf16 subnormals, exact powers of two
    x[0, :128] *= np.float32(2.0 ** -120)
    x[1, 128:256] = np.float32(2.0 ** -130) * np.arange(128, dtype=np.float32)
    x[2, 256:384] = np.float32(448.0 * 2.0 ** -60) * np.sign(x[2, 256:384])
    x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x))
    q, s = blockquant.act_quant(x)
    for m in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            s_exp, codes = rational_group(x[m, 128 * g:128 * (g + 1)].tolist())
            assert Fraction(float(s[m, g])) == s_exp, (m, g)
            assert q[m, 128 * g:128 * (g + 1)].tolist() == codes, (m, g)


def test_max_element_saturates_to_448():
    x = workloads.activations(64, 1024, key=(0, 0, 0, 0))
    q, s = blockquant.act_quant(x)
    xf = workloads.bf16_bits_to_f32(x).reshape(64, 8, 128)
    qg = q.reshape(64, 8, 128)
    idx = np.argmax(np.abs(xf), axis=2)
    top = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_qdq_error_half_ulp():
    x = workloads.activations(32, 2048, key=(0, 1, 0, 0))
    q, s = blockquant.act_quant(x)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    sx = np.repeat(s.astype(np.float64), 128, axis=1)
    r = xf / sx                                   # exact quotient (float64 is close enough:
    d = fp8.dec_e4m3(q)                           # the bound below has slack of 2^-24 |r|)
    a = np.abs(d)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    ulp = 2.0 ** (e - 3)
    # the code brackets r within half an E4M3 ulp of its own binade (plus fp32 rounding of r)
    assert np.all(np.abs(d - r) <= 0.5 * np.maximum(ulp, 2.0 ** -9) + 2.0 ** -23 * np.abs(r) + 1e-300)
    assert np.all(np.abs(d * sx - xf) <= (0.5 * np.maximum(ulp, 2.0 ** -9) + 2.0 ** -23 * np.abs(r)) * sx)


@pytest.mark.parametrize("k", [-20, -3, 1, 7, 30])
def test_power_of_two_scaling(k):
    x = workloads.bf16_bits_to_f32(workloads.activations(8, 512, key=(0, 2, 0, 0)))
    q0, s0 = blockquant.act_quant(x)
    q1, s1 = blockquant.act_quant(x * np.float32(2.0 ** k))
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


def test_row_permutation_and_group_independence():
    x = workloads.activations(16, 768, key=(0, 3, 0, 0))
    q, s = blockquant.act_quant(x)
    perm = np.random.default_rng(0).permutation(16)
    qp, sp = blockquant.act_quant(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    # changing one group leaves the others untouched
    y = x.copy()
    y[:, 256:384] = workloads.activations(16, 128, key=(0, 3, 1, 0))
    qy, sy = blockquant.act_quant(y)
    keep = np.r_[0:256, 384:768]
    assert np.array_equal(qy[:, keep], q[:, keep])
    assert np.array_equal(np.delete(sy, 2, axis=1), np.delete(s, 2, axis=1))


def test_weight_quant_blocks_f32():
    w = workloads.weights(256, 384, key=(0, 5, 1, 0))
    q, s = blockquant.weight_quant(w, "f32")
    assert s.shape == (2, 3) and s.dtype == np.float32
    wf = workloads.bf16_bits_to_f32(w)
    # each block equals act_quant applied to the block flattened as one group of 16384
    for nb in range(2):
        for kb in range(3):
            blk = wf[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)]
            qb, sb = blockquant.act_quant(blk.reshape(1, -1), group=128 * 128)
            assert sb[0, 0] == s[nb, kb]
            assert np.array_equal(qb.reshape(128, 128), q[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)])
            assert (np.abs(fp8.dec_e4m3(q[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)])).max()) == 448.0


def test_weight_quant_ue8m0_exact_division():
    w = workloads.weights(256, 256, key=(0, 6, 1, 0))
    q, s = blockquant.weight_quant(w, "ue8m0")
    assert s.dtype == np.uint8
    wf = workloads.bf16_bits_to_f32(w).astype(np.float64)
    sv = fp8.dec_ue8m0(s)
    sfull = np.repeat(np.repeat(sv, 128, 0), 128, 1)
    r = wf / sfull  # exact: powers of two
    # codes are the RNE E4M3 of the exact quotient; the block maximum stays within (224, 448]
    assert np.array_equal(q, fp8.enc_e4m3_sat(r))
    amax = np.abs(wf).reshape(2, 128, 2, 128).max(axis=(1, 3))
    assert np.all(amax / sv <= 448) and np.all(amax / sv > 224)


def test_ragged_k_last_group():
    x = workloads.activations(4, 300, key=(0, 7, 0, 0))
    q, s = blockquant.act_quant(x)
    assert q.shape == (4, 300) and s.shape == (4, 3)
    s_exp, codes = rational_group(workloads.bf16_bits_to_f32(x)[2, 256:300].tolist())
    assert Fraction(float(s[2, 2])) == s_exp and q[2, 256:300].tolist() == codes
