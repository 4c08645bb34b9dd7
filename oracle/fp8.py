"""Reference fp8 codecs: E4M3, E5M2 and UE8M0 (test infrastructure, CPU, numpy).

Sources
-------
* vLLM "FP8 W8A8" page, section "Two FP8 representations": E4M3 has 1 sign, 4 exponent and
  3 mantissa bits, reaches +-448 and has NaN; E5M2 has 1/5/2 bits, reaches +-57344 and has
  +-inf and NaN.
* SqueezeBits "FP8 Quantization with OwLite", section "What is FP8 format": both formats
  follow IEEE-754 conventions.  Reading: IEEE-style gradual underflow, sign-magnitude, and the
  exponent bias that puts the stated maximum at the top of the finite range.  For E4M3 the
  maximum 448 = 1.75 * 2^8 with no infinity means exponent field 15 holds finite values and
  only mantissa 111 there is NaN, so the bias is 7.  For E5M2, 57344 = 1.75 * 2^15 with
  exponent field 31 reserved for inf/NaN gives bias 15.
* Transformers "Fine-grained FP8", section "UE8M0 scale format": weight scales may be stored as
  float8_e8m0fnu: unsigned, 8 exponent bits, no mantissa.  Reading: bias 127, 0xFF is NaN,
  no zero and no infinity, so code c means 2^(c-127).

Everything here is computed exactly in float64 from the bit fields.  Encoders take finite
values; rounding is to nearest with ties to the even code, and the E4M3 encoder saturates to
+-448 (the rounding and saturation rule this library fixes for quantization).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


# --------------------------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------------------------
def dec_e4m3(codes) -> np.ndarray:
    """u8 E4M3 codes -> float64.  Field layout s|eeee|mmm, bias 7, subnormals at e == 0."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nor)
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val.astype(np.float64)


def dec_e5m2(codes) -> np.ndarray:
    """u8 E5M2 codes -> float64.  Field layout s|eeeee|mm, bias 15; e == 31: inf (m=0) / NaN."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 2) & 0x1F
    m = c & 0x3
    sub = (m / 4.0) * 2.0 ** -14
    nor = (1.0 + m / 4.0) * np.exp2((e - 15).astype(np.float64))
    mag = np.where(e == 0, sub, nor)
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    val = np.where(s == 1, -mag, mag)
    return val.astype(np.float64)


def dec_ue8m0(codes) -> np.ndarray:
    """u8 UE8M0 codes -> float64: 2^(c-127); 0xFF -> NaN."""
    c = np.asarray(codes).astype(np.int64)
    val = np.exp2((c - 127).astype(np.float64))
    return np.where(c == 255, np.nan, val)


# --------------------------------------------------------------------------------------------
# encode
# --------------------------------------------------------------------------------------------
def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0 exactly (via frexp: a = f * 2^x, f in [0.5, 1))."""
    _, x = np.frexp(a)
    return x.astype(np.int64) - 1


def enc_e4m3_sat(r) -> np.ndarray:
    """Finite float (float32 or float64) -> u8 E4M3 code; RNE, saturating to +-448.

    The sign comes from the sign bit, so -0 and negatives that round to zero give 0x80.
    Method: with e = max(floor(log2|r|), -6), t = |r| * 2^(3-e) is exact and lies in [8, 16)
    (or [0, 8) in the subnormal range); rounding t half-to-even to an integer n gives the code
    (e + 6) * 8 + n, where n == 16 carries into the next binade by itself.
    """
    r = np.asarray(r, dtype=np.float64)
    if not np.all(np.isfinite(r)):
        raise ValueError("enc_e4m3_sat: non-finite input is outside the contract")
    neg = np.signbit(r).astype(np.int64)
    a = np.abs(r)
    e = np.full(a.shape, -6, dtype=np.int64)
    nz = a > 0
    e[nz] = np.maximum(_floor_log2(a[nz]), -6)
    t = a * np.exp2((3 - e).astype(np.float64))
    n = np.rint(t).astype(np.int64)  # numpy rint: round half to even
    code = (e + 6) * 8 + n
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.minimum(code, 0x7E)  # a < 448 never exceeds 0x7E; kept as a guard
    return (code | (neg << 7)).astype(np.uint8)


def enc_e5m2(r, saturate: bool = True) -> np.ndarray:
    """Float -> u8 E5M2 code; RNE.

    saturate=True: |r| >= 57344 (inf included) -> 0x7B | sign.
    saturate=False: |r| >= 61440 (the midpoint to 2^16, which rounds to the even code, inf)
    -> inf (0x7C | sign); NaN -> 0x7F | sign.
    """
    r = np.asarray(r, dtype=np.float64)
    neg = np.signbit(r).astype(np.int64)
    nan = np.isnan(r)
    a = np.where(nan, 0.0, np.abs(r))
    fin = np.isfinite(a)
    af = np.where(fin, a, 0.0)
    e = np.full(a.shape, -14, dtype=np.int64)
    nz = af > 0
    e[nz] = np.maximum(_floor_log2(af[nz]), -14)
    t = af * np.exp2((2 - e).astype(np.float64))
    n = np.rint(t).astype(np.int64)
    code = (e + 14) * 4 + n
    if saturate:
        code = np.where(a >= E5M2_MAX, 0x7B, code)
    else:
        code = np.where(a >= 61440.0, 0x7C, code)
    code = np.where(nan, 0x7F, code)
    return (code | (neg << 7)).astype(np.uint8)


def ue8m0_from_amax(amax) -> np.ndarray:
    """Smallest power of two 2^e >= amax/448 (exact), as a UE8M0 code e + 127 clamped to 0..254.

    With amax = f * 2^p, f in [1, 2): amax/448 = (f/1.75) * 2^(p-8), so e = p - 8 when
    f <= 1.75 and p - 7 otherwise.  amax == 0 gives code 127 (scale 1).
    """
    a = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("ue8m0_from_amax: amax must be finite and >= 0")
    f, x = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2^x, f in [0.5, 1)
    p = x.astype(np.int64) - 1                 # a = (2f) * 2^p, 2f in [1, 2)
    e = p - 8 + ((2.0 * f) > 1.75).astype(np.int64)
    code = np.clip(e + 127, 0, 254)
    code = np.where(a > 0, code, 127)
    return code.astype(np.uint8)
