"""Reference for the other FP8 scaling schemes the pages name (test infrastructure, CPU, numpy).

* FP8_DYNAMIC (vLLM "FP8 W8A8", "Quantization process"): weights static and per channel (one
  scale per output feature, i.e. per row of W [N, K]), activations dynamic and per token (one
  scale per row of x over the whole K), plain round-to-nearest.
* Static activation quantization (Transformers "Fine-grained FP8", "DeepGEMM fast path"): the
  activation scale is fixed beforehand instead of computed per call.  Reading: one float32 scale
  for the whole tensor, given by the caller (choosing it needs calibration data, which is out of
  scope); codes are E(fl32(x / s)) with the same rounding and saturation as the dynamic scheme.
* E5M2 operands (vLLM "FP8 W8A8", "Two FP8 representations"): the same schemes with the 1/5/2
  format, whose maximum 57344 takes the place of 448 in every scale.

The GEMM is y[m, n] = a(m) * sum_kb w_kb(n) * P_kb[m, n] where P_kb is the exact product sum of
the decoded codes over K-block kb, a(m) the activation scale (per token or the tensor's one
scale), and w_kb(n) the weight scale (s_w[n] for every kb per channel, or s_w[n // 128, kb] per
128 x 128 block).  Decoded E4M3 values are multiples of 2^-9 and E5M2 values multiples of 2^-16
below 2^16, so every product is exact in float64; a sum of up to 32768 of them may round in
float64, by far less than any tolerance here.
"""
from __future__ import annotations

import numpy as np

from . import blockquant, fp8

GROUP = 128


def _dec(codes, code: str) -> np.ndarray:
    if code == "e4m3":
        return fp8.dec_e4m3(codes)
    if code == "e5m2":
        return fp8.dec_e5m2(codes)
    raise ValueError("code must be 'e4m3' or 'e5m2'")


def token_quant(x, code: str = "e4m3"):
    """Dynamic per-token activation quantization: one group spanning each whole row.

    Returns (q uint8 [M, K], s float32 [M]) with s = fl32(amax_row / max)."""
    K = np.asarray(x).shape[1]
    q, s = blockquant.act_quant(x, group=K, code=code)
    return q, np.ascontiguousarray(s[:, 0])


def channel_weight_quant(w, code: str = "e4m3"):
    """Static per-output-channel weight quantization (one scale per row of W [N, K]), the same
    rule as token_quant applied to the rows of W.  Returns (q uint8 [N, K], s float32 [N])."""
    return token_quant(w, code)


def static_quant(x, s, code: str = "e4m3") -> np.ndarray:
    """Quantization with a given per-tensor scale s (float32, > 0): q = E(fl32(x / s)), RNE,
    saturating.  x: bf16 bits uint16 [M, K] or float32."""
    xf = np.asarray(x)
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    s = np.float32(s)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("static_quant: the scale must be finite and positive")
    if not np.all(np.isfinite(xf)):
        raise ValueError("static_quant: non-finite input is outside the contract")
    r = (xf / s).astype(np.float32)  # one IEEE float32 division per element
    return np.ascontiguousarray(blockquant.encode(r, code))


def scaled_gemm_ref(a_q, a_scale, w_q, w_scale, *, act: str, weight: str, a_code: str = "e4m3",
                    w_code: str = "e4m3", w_scale_fmt: str = "f32") -> np.ndarray:
    """y = a(m) * sum_kb w_kb(n) * P_kb in float64.

    act "token": a_scale float32 [M]; "tensor": a_scale float32 scalar.
    weight "channel": w_scale float32 [N]; "block": w_scale [N/128, K/128] float32 or UE8M0
    codes (w_scale_fmt).  Returns float64 [M, N]."""
    M, K = a_q.shape
    N = w_q.shape[0]
    A = _dec(a_q, a_code)
    W = _dec(w_q, w_code)
    if act == "token":
        am = np.asarray(a_scale, dtype=np.float32).astype(np.float64).reshape(M)
    elif act == "tensor":
        am = np.full(M, float(np.float32(a_scale)), dtype=np.float64)
    else:
        raise ValueError("act must be 'token' or 'tensor'")
    if weight == "channel":
        wn = np.asarray(w_scale, dtype=np.float32).astype(np.float64).reshape(N)
        y = A @ W.T
        return am[:, None] * y * wn[None, :]
    if weight != "block":
        raise ValueError("weight must be 'channel' or 'block'")
    if w_scale_fmt == "f32":
        sw = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    elif w_scale_fmt == "ue8m0":
        sw = fp8.dec_ue8m0(np.asarray(w_scale, dtype=np.uint8))
    else:
        raise ValueError("w_scale_fmt must be 'f32' or 'ue8m0'")
    sw_cols = np.repeat(sw, GROUP, axis=0)[:N]  # [N, KB]
    y = np.zeros((M, N), dtype=np.float64)
    for kb in range(-(-K // GROUP)):
        k0, k1 = kb * GROUP, min(K, (kb + 1) * GROUP)
        y += (A[:, k0:k1] @ W[:, k0:k1].T) * sw_cols[None, :, kb]
    return am[:, None] * y
