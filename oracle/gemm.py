"""Reference block-scaled W8A8 GEMM and its grouped (MoE) variant (test infrastructure, CPU).

Transformers "Fine-grained FP8", section "DeepGEMM fast path": every FP8 linear with
(128, 128) weight blocks and dynamic activations runs one block-scaled FP8 GEMM; MoE expert
matmuls have their own grouped backends (same page, "DeepGEMM fast path" and "UE8M0 scale
format").  vLLM "FP8 W8A8", intro: both operands are 8-bit (W8A8).

The layer computes, with y = A . W^T (the PyTorch Linear layout, W is [N, K]):

    y[m, n] = sum_kb  s_a[m, kb] * s_w[n // 128, kb] * sum_{k in kb} dec(A_q[m, k]) * dec(W_q[n, k])

Every decoded E4M3 value is an integer multiple of 2^-9 below 2^9 in magnitude, so each
product is a multiple of 2^-18 and a sum of up to 128 of them is an integer multiple of 2^-18
below 2^43 in magnitude: the per-block partial sums P_kb are exact in float64 whatever the
summation order.  The scaled sum over blocks is then taken in float64, in ascending kb.
"""
from __future__ import annotations

import numpy as np

from . import fp8

GROUP = 128


def _w_scales(s_w, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.asarray(s_w, dtype=np.float32).astype(np.float64)
    if fmt == "ue8m0":
        return fp8.dec_ue8m0(np.asarray(s_w, dtype=np.uint8))
    raise ValueError("fmt must be 'f32' or 'ue8m0'")


def gemm_ref(a_q, s_a, w_q, s_w, fmt: str = "f32") -> np.ndarray:
    """Exact-partial block-scaled GEMM in float64.

    a_q uint8 [M, K]; s_a float32 [M, KB] (logical layout); w_q uint8 [N, K];
    s_w [NB, KB] float32 or UE8M0 codes.  Returns float64 [M, N].
    """
    M, K = a_q.shape
    N = w_q.shape[0]
    KB = -(-K // GROUP)
    A = fp8.dec_e4m3(a_q)
    W = fp8.dec_e4m3(w_q)
    sa = np.asarray(s_a, dtype=np.float32).astype(np.float64)
    sw = _w_scales(s_w, fmt)
    sw_cols = np.repeat(sw, GROUP, axis=0)[:N]  # [N, KB]: scale of output column n
    y = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        k0, k1 = kb * GROUP, min(K, (kb + 1) * GROUP)
        P = A[:, k0:k1] @ W[:, k0:k1].T  # exact (see module docstring)
        y += (sa[:, kb, None] * sw_cols[None, :, kb]) * P
    return y


def gemm_ref_fast(a_q, s_a, w_q, s_w, fmt: str = "f32") -> np.ndarray:
    """One float64 GEMM of the fully dequantized operands.

    Not exact (the scales are folded in before summation), but within ~1e-15 relative of
    gemm_ref; used only to bound the oracle's time on large shapes.
    """
    M, K = a_q.shape
    N = w_q.shape[0]
    sa = np.asarray(s_a, dtype=np.float32).astype(np.float64)
    sw = _w_scales(s_w, fmt)
    A = fp8.dec_e4m3(a_q) * np.repeat(sa, GROUP, axis=1)[:, :K]
    sw_full = np.repeat(np.repeat(sw, GROUP, axis=0)[:N], GROUP, axis=1)[:, :K]
    W = fp8.dec_e4m3(w_q) * sw_full
    return A @ W.T


def grouped_ref(a_q, s_a, w_q, s_w, offsets, fmt: str = "f32", fast: bool = False) -> np.ndarray:
    """Per-expert block-scaled GEMM over contiguous row ranges.

    a_q [total_M, K]; s_a [total_M, KB]; w_q [E, N, K]; s_w [E, NB, KB];
    offsets int [E+1], nondecreasing from 0 to total_M.  Rows of expert e are
    offsets[e] .. offsets[e+1]-1.  Returns float64 [total_M, N].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = w_q.shape[0]
    total_M = a_q.shape[0]
    N = w_q.shape[1]
    if offsets.shape != (E + 1,) or offsets[0] != 0 or offsets[-1] != total_M or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be nondecreasing from 0 to total_M with E+1 entries")
    f = gemm_ref_fast if fast else gemm_ref
    y = np.zeros((total_M, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            y[r0:r1] = f(a_q[r0:r1], s_a[r0:r1], w_q[e], s_w[e], fmt)
    return y


def bf16_rne(y) -> np.ndarray:
    """Round float64 values directly to bf16 (nearest, ties to even); returns float64 values.

    bf16 keeps 8 significant bits and float32's exponent range.  Values beyond the largest
    finite bf16 after rounding become inf; gradual underflow below 2^-126.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    a = np.abs(y)
    nz = a > 0
    _, x = np.frexp(a[nz])                     # a = f * 2^x, f in [0.5, 1)
    x = np.maximum(x.astype(np.int64), -125)   # below 2^-126: fixed quantum 2^-133
    q = np.exp2((x - 8).astype(np.float64))    # quantum of the binade
    out[nz] = np.rint(a[nz] / q) * q           # exact: division by a power of two
    out = np.where(out > 3.3895313892515355e38, np.inf, out)
    return np.copysign(out, y)


def batched_ref(a_q, s_a, w_q, s_w, counts, max_m: int, fmt: str = "f32", fast: bool = False):
    """Masked batched layout: expert e owns rows e*max_m .. e*max_m + counts[e] - 1 of a_q
    [E*max_m, K] and s_a [E*max_m, KB]; the remaining rows of its slot are padding.

    Returns (y float64 [E*max_m, N], valid bool [E*max_m]): y holds the per-expert block GEMM on
    the valid rows and 0 on padding rows (whose output is not defined)."""
    counts = np.asarray(counts, dtype=np.int64)
    E = w_q.shape[0]
    N = w_q.shape[1]
    if counts.shape != (E,) or np.any(counts < 0) or np.any(counts > max_m) or a_q.shape[0] != E * max_m:
        raise ValueError("counts must be [E] within 0 .. max_m, a_q [E*max_m, K]")
    f = gemm_ref_fast if fast else gemm_ref
    y = np.zeros((E * max_m, N), dtype=np.float64)
    valid = np.zeros(E * max_m, dtype=bool)
    for e in range(E):
        r0, r1 = e * max_m, e * max_m + counts[e]
        valid[r0:r1] = True
        if r1 > r0:
            y[r0:r1] = f(a_q[r0:r1], s_a[r0:r1], w_q[e], s_w[e], fmt)
    return y, valid

