"""GPU parity: the fp8 codec kernels against the oracle (bit-exact), and the hardware E4M3
conversion against the integer bit-field encoder over every non-NaN float32."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
from oracle import fp8

pytestmark = pytest.mark.gpu

ALL = np.arange(256, dtype=np.uint8)


def _structured_f32(lo_exp=100, hi_exp=141):
    """Every exponent in [lo, hi) x top-5 mantissa patterns x low-bit patterns around the
    rounding points of 3-bit (E4M3) and 2-bit (E5M2) mantissas, both signs."""
    exps = np.arange(lo_exp, hi_exp, dtype=np.uint32)
    top = np.arange(32, dtype=np.uint32) << 18
    low = np.array([0, 1, 0x1FFFF, 0x20000, 0x20001, 0x3FFFF, 0x0FFFF, 0x10000, 0x10001, 0x2AAAA], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | top[None, :, None] | low[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def _bf16_all_finite():
    b = np.arange(0x10000, dtype=np.uint32)
    b = b[((b & 0x7F80) != 0x7F80)]
    return (b << 16).view(np.float32)


def _inputs():
    rng = np.random.default_rng(21)
    parts = [
        _structured_f32(),
        _bf16_all_finite(),
        rng.uniform(-600, 600, 1 << 20).astype(np.float32),
        (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-30, 10, 1 << 20))).astype(np.float32),
        np.float32([0.0, -0.0, 448.0, -448.0, 464.0, 463.99997, 1e38, -1e38, np.inf, -np.inf]),
    ]
    return np.concatenate(parts)


def test_decode_all_codes(dev):
    c = torch.from_numpy(ALL.copy()).to(dev)
    for fmt, ref in [(fgb.FP8_E4M3, fp8.dec_e4m3), (fgb.FP8_E5M2, fp8.dec_e5m2), (fgb.UE8M0, fp8.dec_ue8m0)]:
        got = fgb.fp8_decode(c, fmt).cpu().numpy().astype(np.float64)
        exp = ref(ALL)
        assert np.array_equal(got, exp, equal_nan=True), fmt
        num = ~np.isnan(exp)  # the sign of a NaN carries no meaning
        assert np.array_equal(np.signbit(got[num]), np.signbit(exp[num])), fmt


def test_encode_e4m3_hardware_vs_oracle(dev):
    x = _inputs()
    fin = np.isfinite(x)
    got = fgb.fp8_encode(torch.from_numpy(x).to(dev), fgb.FP8_E4M3).cpu().numpy()
    exp = fp8.enc_e4m3_sat(x[fin])
    assert np.array_equal(got[fin], exp)
    # +-inf saturate like any other out-of-range value
    assert got[~fin].tolist() == [0x7E, 0xFE]


def test_encode_e4m3_integer_vs_oracle(dev):
    x = _inputs()
    x = x[np.isfinite(x)]
    got = fgb.fp8_encode(torch.from_numpy(x).to(dev), fgb.FP8_E4M3_INT).cpu().numpy()
    assert np.array_equal(got, fp8.enc_e4m3_sat(x))


def test_encode_e4m3_hardware_equals_integer_on_every_float32(dev):
    """All 2^32 bit patterns except NaNs, in chunks of 2^28, generated on the device."""
    chunk = 1 << 28
    mism = 0
    for start in range(0, 1 << 32, chunk):
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device=dev).to(torch.int32)
        x = bits.view(torch.float32)
        hw = fgb.fp8_encode(x, fgb.FP8_E4M3)
        sw = fgb.fp8_encode(x, fgb.FP8_E4M3_INT)
        nan = torch.isnan(x)
        mism += int(((hw != sw) & ~nan).sum().item())
        del bits, x, hw, sw, nan
    torch.cuda.synchronize()
    assert mism == 0


@pytest.mark.parametrize("sat", [True, False])
def test_encode_e5m2_vs_oracle(dev, sat):
    x = _inputs()
    x = np.concatenate([x[np.isfinite(x)], np.float32([57344.0, 61439.996, 61440.0, 65536.0, -61440.0])])
    got = fgb.fp8_encode(torch.from_numpy(x).to(dev), fgb.FP8_E5M2, saturate=sat).cpu().numpy()
    assert np.array_equal(got, fp8.enc_e5m2(x, saturate=sat))


def test_encode_ue8m0_vs_oracle(dev):
    b = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    a = np.concatenate([(b << 16).view(np.float32),
                        np.abs(np.random.default_rng(3).standard_normal(1 << 20)).astype(np.float32) * np.float32(1e3)])
    got = fgb.fp8_encode(torch.from_numpy(a).to(dev), fgb.UE8M0).cpu().numpy()
    assert np.array_equal(got, fp8.ue8m0_from_amax(a))
