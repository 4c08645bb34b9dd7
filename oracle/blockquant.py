"""Reference fine-grained FP8 quantization (test infrastructure, CPU, numpy).

Transformers "Fine-grained FP8", intro: weights are quantized to 8 bits per 2-D block
(weight_block_size = (128, 128)); activations are quantized to 8 bits per token, per group,
where the group equals the weight block along input channels (128).  Section "DeepGEMM fast
path": the activation scheme is dynamic, i.e. activation scales are computed at run time.

Readings fixed by this library where the pages leave a step open:
* The scale is the AbsMax of the group (OwLite page, "FP8 format support in TensorRT", names
  AbsMax calibration) divided by the E4M3 maximum 448 (vLLM "FP8 W8A8", "Two FP8
  representations"): s = fl32(amax / 448), one IEEE float32 division.
* Codes are q = enc_e4m3_sat(fl32(x / s)): an IEEE float32 division by the stored scale, then
  round-to-nearest-even with saturation to +-448.
* A group whose amax is 0 gets s = 0 and codes +-0 by the sign of x.
* With UE8M0 weight scales (Transformers "Fine-grained FP8", "UE8M0 scale format") the scale
  is the smallest power of two >= amax/448, so x / s is exact.
"""
from __future__ import annotations

import numpy as np

from . import fp8

GROUP = 128


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns: widen exactly
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype != np.float32:
        raise TypeError("expected bf16 bits (uint16) or float32 values")
    return x


# the largest finite value of each code format (vLLM "FP8 W8A8", "Two FP8 representations")
CODE_MAX = {"e4m3": np.float32(448.0), "e5m2": np.float32(57344.0)}


def encode(r, code: str = "e4m3") -> np.ndarray:
    """Round-to-nearest-even, saturating encoder of the chosen format."""
    if code == "e4m3":
        return fp8.enc_e4m3_sat(r)
    if code == "e5m2":
        return fp8.enc_e5m2(r, saturate=True)
    raise ValueError("code must be 'e4m3' or 'e5m2'")


def _quantize_groups(xg: np.ndarray, s: np.ndarray, code: str = "e4m3") -> np.ndarray:
    """xg float32 [..., G, L]; s float32 [..., G] -> u8 codes [..., G, L]."""
    with np.errstate(divide="ignore", invalid="ignore"):
        r = xg / s[..., None]  # float32 / float32: IEEE correctly rounded
    zero = (s == 0)[..., None] & np.ones(xg.shape, dtype=bool)
    r = np.where(zero, 0.0, r)
    q = encode(r, code)
    # amax == 0: every element is +-0; keep its sign (enc saw +0 after the where above)
    signs = (np.signbit(xg).astype(np.uint8) << 7)
    return np.where(zero, signs, q).astype(np.uint8)


def act_quant(x, group: int = GROUP, code: str = "e4m3"):
    """Dynamic per-token, per-group activation quantization.

    x: bf16 bits uint16 [M, K] (or float32 holding bf16-exact values), finite.
    Returns (q uint8 [M, K], s float32 [M, ceil(K/group)]).  The last group may be partial.
    s = fl32(amax / max) with max = 448 for E4M3 codes, 57344 for E5M2 codes.
    """
    xf = _as_f32(x)
    if not np.all(np.isfinite(xf)):
        raise ValueError("act_quant: non-finite input is outside the contract")
    M, K = xf.shape
    G = -(-K // group)
    pad = G * group - K
    xp = np.pad(xf, ((0, 0), (0, pad))) if pad else xf
    xg = xp.reshape(M, G, group)
    amax = np.max(np.abs(xg), axis=2)                 # exact
    s = (amax / CODE_MAX[code]).astype(np.float32)     # one IEEE float32 division
    q = _quantize_groups(xg, s, code).reshape(M, G * group)[:, :K]
    return np.ascontiguousarray(q), s


def weight_quant(w, fmt: str = "f32", block: int = GROUP, code: str = "e4m3"):
    """Per 128x128 block weight quantization.

    w: bf16 bits uint16 [N, K] (or float32).  fmt: "f32" -> s float32 [ceil(N/128), ceil(K/128)];
    "ue8m0" -> s uint8 UE8M0 codes of the same shape (E4M3 codes only).  code: "e4m3" or
    "e5m2" (float32 scales amax / 57344).
    Returns (q uint8 [N, K], s).
    """
    if fmt == "ue8m0" and code != "e4m3":
        raise ValueError("UE8M0 weight scales go with E4M3 codes")
    wf = _as_f32(w)
    if not np.all(np.isfinite(wf)):
        raise ValueError("weight_quant: non-finite input is outside the contract")
    N, K = wf.shape
    NB, KB = -(-N // block), -(-K // block)
    wp = np.pad(wf, ((0, NB * block - N), (0, KB * block - K)))
    blocks = wp.reshape(NB, block, KB, block).transpose(0, 2, 1, 3)  # [NB, KB, b, b]
    amax = np.max(np.abs(blocks), axis=(2, 3))
    if fmt == "f32":
        s = (amax / CODE_MAX[code]).astype(np.float32)
        s_used = s
    elif fmt == "ue8m0":
        s = fp8.ue8m0_from_amax(amax)
        s_used = fp8.dec_ue8m0(s).astype(np.float32)  # powers of two, exact in float32
    else:
        raise ValueError("fmt must be 'f32' or 'ue8m0'")
    flat = blocks.reshape(NB, KB, block * block)
    q = _quantize_groups(flat, s_used, code).reshape(NB, KB, block, block)
    q = q.transpose(0, 2, 1, 3).reshape(NB * block, KB * block)[:N, :K]
    return np.ascontiguousarray(q), s

