"""Pins for the oracle's fp8 codecs (CPU).

What fixes the answers, independently of the oracle's own method:
* the formats' printed facts (vLLM "FP8 W8A8", "Two FP8 representations"): E4M3 reaches
  +-448 and has NaN but no inf; E5M2 reaches +-57344 and has +-inf and NaN;
* torch's float8_e4m3fn / float8_e5m2 / float8_e8m0fnu dtypes as a library decode table, and
  torch's float32 -> fp8 cast (round-to-nearest-even) on its in-range branch;
* brute-force nearest-value searches over the decoded tables (ties to the even code);
* closed forms for the power-of-two UE8M0 scale.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(dtype):
    return torch.from_numpy(ALL.copy()).view(dtype).double().numpy()


# ------------------------------------------------------------------------------------------
# decode tables
# ------------------------------------------------------------------------------------------
def test_e4m3_printed_facts():
    d = fp8.dec_e4m3(ALL)
    fin = np.isfinite(d)
    assert np.nanmax(d) == 448.0 and np.nanmin(d) == -448.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert set(ALL[np.isnan(d)].tolist()) == {0x7F, 0xFF}
    assert not np.any(np.isinf(d))
    assert fin.sum() == 254
    # IEEE-style gradual underflow: smallest positive value 2^-9, smallest normal 2^-6
    pos = d[(d > 0) & fin]
    assert pos.min() == 2.0 ** -9
    assert d[0x08] == 2.0 ** -6 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x38] == 1.0  # exponent field 7 == bias
    assert d[0x00] == 0.0 and not np.signbit(d[0x00]) and np.signbit(d[0x80])


def test_e4m3_matches_torch_table():
    assert np.array_equal(fp8.dec_e4m3(ALL), _torch_decode(torch.float8_e4m3fn), equal_nan=True)


def test_e4m3_monotone_per_sign():
    d = fp8.dec_e4m3(ALL)
    assert np.all(np.diff(d[0x00:0x7F]) > 0)
    assert np.all(np.diff(d[0x80:0xFF]) < 0)
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])


def test_e5m2_printed_facts():
    d = fp8.dec_e5m2(ALL)
    assert np.nanmax(d[np.isfinite(d)]) == 57344.0 and d[0x7B] == 57344.0 and d[0xFB] == -57344.0
    assert d[0x7C] == np.inf and d[0xFC] == -np.inf
    assert set(ALL[np.isnan(d)].tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert np.isfinite(d).sum() == 248
    assert d[(d > 0) & np.isfinite(d)].min() == 2.0 ** -16
    assert d[0x3C] == 1.0


def test_e5m2_matches_torch_table():
    assert np.array_equal(fp8.dec_e5m2(ALL), _torch_decode(torch.float8_e5m2), equal_nan=True)


def test_ue8m0_table_closed_form_and_torch():
    d = fp8.dec_ue8m0(ALL)
    assert np.array_equal(d, _torch_decode(torch.float8_e8m0fnu), equal_nan=True)
    f32 = d[1:255].astype(np.float32)
    assert np.array_equal(f32.view(np.uint32), (ALL[1:255].astype(np.uint32) << 23))
    assert d[0] == 2.0 ** -127 and np.isnan(d[255]) and d[127] == 1.0


# ------------------------------------------------------------------------------------------
# brute-force encoders (nearest value in the decoded table, ties to the even code)
# ------------------------------------------------------------------------------------------
def _brute_nearest(r, table_codes, table_vals, max_code):
    """Nearest magnitude code by exhaustive search; ties -> code with LSB 0; |r| >= max -> max."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    dist = np.abs(a[:, None] - table_vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer the even code
    even = (table_codes[None, :] & 1) == 0
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, np.argmax(pick_even, axis=1), np.argmax(cand, axis=1))
    code = table_codes[idx]
    code = np.where(a >= table_vals.max(), max_code, code)
    return (code | (np.signbit(r).astype(np.int64) << 7)).astype(np.uint8)


def _e4m3_pos_table():
    codes = np.arange(0x00, 0x7F, dtype=np.int64)  # +0 .. 448
    return codes, fp8.dec_e4m3(codes)


def _probes(vals, rng, lo, hi, n_rand=200000):
    """Midpoints between neighbours, fp32 neighbours of midpoints and values, random draws."""
    v = np.unique(vals)
    mids = (v[:-1] + v[1:]) / 2
    base = np.concatenate([v, mids]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    rnd_lin = rng.uniform(lo, hi, n_rand).astype(np.float32)
    rnd_log = (np.exp2(rng.uniform(np.log2(lo if lo > 0 else 2.0 ** -30), np.log2(hi), n_rand))).astype(np.float32)
    p = np.concatenate([base, up, dn, rnd_lin, rnd_log])
    p = p[np.isfinite(p)]
    return np.concatenate([p, -p])


def test_enc_e4m3_roundtrip_all_finite_codes():
    d = fp8.dec_e4m3(ALL)
    fin = np.isfinite(d)
    assert np.array_equal(fp8.enc_e4m3_sat(d[fin]), ALL[fin])


def test_enc_e4m3_bruteforce():
    rng = np.random.default_rng(11)
    codes, vals = _e4m3_pos_table()
    probes = _probes(vals, rng, 0.0, 600.0)
    probes = np.concatenate([probes, np.float32([1e30, -1e30, 465.0, 464.0, 463.99997, 448.00003, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -10, 2.0 ** -10 * 1.0000001])])
    for chunk in np.array_split(probes, 40):
        exp = _brute_nearest(chunk, codes, vals, 0x7E)
        got = fp8.enc_e4m3_sat(chunk)
        bad = np.nonzero(exp != got)[0]
        assert bad.size == 0, (chunk[bad[:5]], exp[bad[:5]], got[bad[:5]])


def test_enc_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.uniform(-463.9, 463.9, 500000), rng.standard_normal(500000) * 1e-2]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.enc_e4m3_sat(x), t)


def test_enc_e4m3_signed_zero_and_underflow():
    assert fp8.enc_e4m3_sat(np.float32([-0.0]))[0] == 0x80
    assert fp8.enc_e4m3_sat(np.float32([0.0]))[0] == 0x00
    assert fp8.enc_e4m3_sat(np.float32([-(2.0 ** -11)]))[0] == 0x80
    # exactly half the smallest subnormal ties to the even code (zero)
    assert fp8.enc_e4m3_sat(np.float32([2.0 ** -10]))[0] == 0x00
    assert fp8.enc_e4m3_sat(np.float32([3 * 2.0 ** -10]))[0] == 0x02


def test_enc_e4m3_saturates():
    big = np.float32([448.0, 449.0, 464.0, 1e38, -500.0, -448.0])
    assert fp8.enc_e4m3_sat(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    with pytest.raises(ValueError):
        fp8.enc_e4m3_sat(np.float32([np.inf]))


def test_enc_e5m2_bruteforce_and_torch():
    rng = np.random.default_rng(13)
    codes = np.arange(0x00, 0x7C, dtype=np.int64)
    vals = fp8.dec_e5m2(codes)
    probes = _probes(vals, rng, 0.0, 60000.0)
    for chunk in np.array_split(probes, 40):
        exp = _brute_nearest(chunk, codes, vals, 0x7B)
        assert np.array_equal(fp8.enc_e5m2(chunk, saturate=True), exp)
    # non-saturating branch against torch's cast (overflow -> inf), all magnitudes
    x = np.concatenate([probes, np.float32([61439.996, 61440.0, 65536.0, 1e30, -61440.0])]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(fp8.enc_e5m2(x, saturate=False), t)
    assert fp8.enc_e5m2(np.float32([np.nan]), saturate=False)[0] & 0x7F == 0x7F
    assert fp8.enc_e5m2(np.float32([np.inf, -np.inf]), saturate=True).tolist() == [0x7B, 0xFB]


# ------------------------------------------------------------------------------------------
# UE8M0 scale choice: the smallest power of two >= amax / 448
# ------------------------------------------------------------------------------------------
def _ue8m0_exact(a: float) -> int:
    if a == 0:
        return 127
    q = Fraction(a) / 448
    e = math.floor(math.log2(q)) - 2
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return int(min(max(e + 127, 0), 254))


def test_ue8m0_from_amax_exact_over_all_bf16():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)  # every positive finite bf16
    amax = (bits << 16).view(np.float32)
    got = fp8.ue8m0_from_amax(amax)
    sample = np.concatenate([np.arange(0, bits.size, 37), np.arange(bits.size - 300, bits.size)])
    for i in sample:
        assert got[i] == _ue8m0_exact(float(amax[i])), float(amax[i])
    s = fp8.dec_ue8m0(got)
    ratio = amax.astype(np.float64) / s
    normal = got > 0  # no clamping at the bottom
    assert np.all(ratio[normal] <= 448.0) and np.all(ratio[normal] > 224.0)


def test_ue8m0_worked_values():
    a = np.float32([448.0, 449.0, 224.0, 1.0, 0.0, 896.0, 447.0])
    assert fp8.ue8m0_from_amax(a).tolist() == [127, 128, 126, 119, 127, 128, 127]
