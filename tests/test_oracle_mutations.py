"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each one.

Each mutant replaces one oracle function with a subtly wrong variant (a wrong bias, ties away
from zero, a lost sign, multiply-by-reciprocal, a transposed scale index, a dropped K-block,
floor instead of ceil); the listed pin must then fail.
"""
import numpy as np
import pytest

from oracle import blockquant, fp8, gemm, schemes
import tests.test_oracle_fp8 as T8
import tests.test_oracle_gemm as TG
import tests.test_oracle_quant as TQ
import tests.test_oracle_schemes as TS

_orig_dec = fp8.dec_e4m3
_orig_enc = fp8.enc_e4m3_sat
_orig_gemm = gemm.gemm_ref


def _dec_bias8(codes):
    v = _orig_dec(codes)
    c = np.asarray(codes).astype(np.int64)
    return np.where(((c >> 3) & 15) > 0, v / 2.0, v)


def _enc_ties_away(r):
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    e = np.full(a.shape, -6, dtype=np.int64)
    nz = a > 0
    e[nz] = np.maximum(np.frexp(a[nz])[1] - 1, -6)
    n = np.floor(a * np.exp2((3 - e).astype(np.float64)) + 0.5).astype(np.int64)
    code = np.minimum(np.where(a >= 448, 0x7E, (e + 6) * 8 + n), 0x7E)
    return (code | (np.signbit(r).astype(np.int64) << 7)).astype(np.uint8)


def _enc_lost_zero_sign(r):
    q = _orig_enc(r)
    return np.where((q & 0x7F) == 0, 0, q).astype(np.uint8)


def _act_quant_reciprocal(x, group=128):
    xf = blockquant._as_f32(x)
    M, K = xf.shape
    xg = xf.reshape(M, K // group, group)
    amax = np.abs(xg).max(axis=2)
    s = (amax / np.float32(448)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = (np.float32(448) / amax).astype(np.float32)
    r = np.where(amax[..., None] > 0, xg * inv[..., None], 0.0).astype(np.float32)
    return _orig_enc(r).reshape(M, K), s


def _act_quant_wrong_max(x, group=128):
    q, s = _orig_act(x, group)
    return q, (s * np.float32(448.0 / 447.0)).astype(np.float32)


_orig_act = blockquant.act_quant


def _gemm_transposed_sw(aq, sa, wq, sw, fmt="f32"):
    sw = np.asarray(sw)
    swt = np.resize(sw.T.reshape(-1), sw.shape)
    return _orig_gemm(aq, sa, wq, swt, fmt)


def _gemm_drop_last_block(aq, sa, wq, sw, fmt="f32"):
    K = aq.shape[1]
    aq2 = aq.copy()
    aq2[:, K - 128:] = 0
    return _orig_gemm(aq2, sa, wq, sw, fmt)


def _ue8m0_floor(amax):
    c = _orig_ue(amax)
    a = np.asarray(amax, np.float64)
    exact = (a > 0) & (fp8.dec_ue8m0(c) * 448.0 != a)
    return np.where(exact, c - 1, c).astype(np.uint8)


_orig_ue = fp8.ue8m0_from_amax

_orig_token = schemes.token_quant
_orig_static = schemes.static_quant
_orig_scaled = schemes.scaled_gemm_ref


def _token_quant_column_amax(x, code="e4m3"):
    """per-channel of x instead of per-token: the scale of column k applied to row k's place"""
    q, s = _orig_token(np.ascontiguousarray(np.asarray(x).T), code)
    return np.ascontiguousarray(q.T), s[: np.asarray(x).shape[0]]


def _static_reciprocal(x, s, code="e4m3"):
    xf = np.asarray(x)
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(s)
    return blockquant.encode((xf * inv).astype(np.float32), code)


def _scaled_channel_by_row(a_q, a_scale, w_q, w_scale, **kw):
    if kw.get("weight") == "channel":
        y = _orig_scaled(a_q, a_scale, w_q, np.ones(w_q.shape[0], np.float32), **kw)
        ws = np.resize(np.asarray(w_scale, np.float64), a_q.shape[0])
        return y * ws[:, None]
    return _orig_scaled(a_q, a_scale, w_q, w_scale, **kw)


def _scaled_tensor_scale_dropped(a_q, a_scale, w_q, w_scale, **kw):
    if kw.get("act") == "tensor":
        return _orig_scaled(a_q, np.float32(1.0), w_q, w_scale, **kw)
    return _orig_scaled(a_q, a_scale, w_q, w_scale, **kw)


_orig_batched = gemm.batched_ref


def _batched_shifted_slots(a_q, s_a, w_q, s_w, counts, max_m, fmt="f32", fast=False):
    """expert e's slot taken to start one row late"""
    a2 = np.roll(a_q, -1, axis=0)
    s2 = np.roll(s_a, -1, axis=0)
    return _orig_batched(a2, s2, w_q, s_w, counts, max_m, fmt, fast)


MUTANTS = [
    ("decode bias 8", fp8, "dec_e4m3", _dec_bias8, [T8.test_e4m3_printed_facts, T8.test_e4m3_matches_torch_table]),
    ("ties away from zero", fp8, "enc_e4m3_sat", _enc_ties_away, [T8.test_enc_e4m3_bruteforce, TQ.test_golden_handworked_groups]),
    ("lost sign of zero", fp8, "enc_e4m3_sat", _enc_lost_zero_sign, [T8.test_enc_e4m3_signed_zero_and_underflow, TQ.test_golden_handworked_groups]),
    ("multiply by reciprocal", blockquant, "act_quant", _act_quant_reciprocal, [TQ.test_division_by_stored_scale_reading]),
    ("scale amax/447", blockquant, "act_quant", _act_quant_wrong_max, [TQ.test_golden_handworked_groups]),
    ("transposed weight-scale index", gemm, "gemm_ref", _gemm_transposed_sw, [lambda: TG.test_blockwise_equals_dense_bruteforce("f32")]),
    ("dropped last K-block", gemm, "gemm_ref", _gemm_drop_last_block, [lambda: TG.test_blockwise_equals_dense_bruteforce("f32"), TG.test_exact_integer_special_case]),
    ("UE8M0 floor instead of ceil", fp8, "ue8m0_from_amax", _ue8m0_floor, [TQ.test_golden_ue8m0_scale_choice]),
    ("per-token scale over columns", schemes, "token_quant", _token_quant_column_amax,
     [lambda: TS.test_token_quant_rational_definition("e4m3"), TS.test_token_quant_reduces_to_group_quant_at_k128]),
    ("static quant by reciprocal", schemes, "static_quant", _static_reciprocal,
     [TS.test_static_quant_divides_by_the_scale]),
    ("channel scale on rows", schemes, "scaled_gemm_ref", _scaled_channel_by_row,
     [TS.test_token_channel_gemm_reduces_to_block_gemm]),
    ("batched slot off by one row", gemm, "batched_ref", _batched_shifted_slots,
     [TG.test_batched_reduces_to_grouped_with_empty_and_full_experts]),
    ("static scale dropped", schemes, "scaled_gemm_ref", _scaled_tensor_scale_dropped,
     [lambda: TS.test_tensor_block_gemm_reduces_to_block_gemm("f32")]),
]


def test_pin_catches_e5m2_maximum_448(monkeypatch):
    monkeypatch.setitem(blockquant.CODE_MAX, "e5m2", np.float32(448.0))
    for pin in (TS.test_e5m2_max_element_reaches_57344, TS.test_e5m2_group_quant_rational_definition):
        with pytest.raises(AssertionError):
            pin()


@pytest.mark.parametrize("name,mod,attr,mutant,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mod, attr, mutant, pins):
    monkeypatch.setattr(mod, attr, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
