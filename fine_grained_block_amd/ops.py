"""torch-tensor wrappers over the C-ABI (argument marshalling only).

Tensors must live on the current HIP device; outputs are allocated with torch and the calls
are enqueued on torch's current stream.  Shapes, strides and enums are validated by the
library itself, which returns a status that is turned into FGBError (a ValueError).
"""
from __future__ import annotations

import torch

from ._lib import FP8_E4M3, OUT_BF16, OUT_F32, SCALE_F32, SCALE_UE8M0, check, lib

BLOCK = 128


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _row_ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit inner stride")
    return t.stride(0)


def _ceil4(n: int) -> int:
    return (n + 3) // 4 * 4


def quantize(x: torch.Tensor, out: tuple | None = None):
    """Dynamic per-token 1x128-group E4M3 quantization of bf16 activations.

    Returns (q uint8 [M, K], s_a float32 [K/128, ld_sa]) with ld_sa = M rounded up to 4;
    s_a[:, :M].t() is the logical [M, K/128] scale matrix.
    """
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize expects bf16 activations")
    M, K = x.shape
    if out is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s_a = torch.empty((K // BLOCK if K % BLOCK == 0 else 0, max(_ceil4(M), 4)), dtype=torch.float32, device=x.device)
    else:
        q, s_a = out
    st = lib().fgb_act_quant_group128(_ptr(x), M, K, _row_ld(x), _ptr(q), _row_ld(q), _ptr(s_a),
                                      s_a.stride(0), _stream())
    check("fgb_act_quant_group128", st)
    return q, s_a


def quantize_weight(w: torch.Tensor, scale_fmt: str = "float"):
    """Per-128x128-block E4M3 weight quantization of a dense bf16 [N, K] matrix.

    scale_fmt "float" -> s_w float32 [N/128, K/128]; "ue8m0" -> s_w uint8 UE8M0 codes.
    """
    if w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError("quantize_weight expects a contiguous bf16 [N, K] tensor")
    N, K = w.shape
    fmt = {"float": SCALE_F32, "ue8m0": SCALE_UE8M0}.get(scale_fmt)
    if fmt is None:
        raise ValueError("scale_fmt must be 'float' or 'ue8m0'")
    w_q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    sdt = torch.float32 if fmt == SCALE_F32 else torch.uint8
    s_w = torch.empty((max(N // BLOCK, 1), max(K // BLOCK, 1)), dtype=sdt, device=w.device)
    st = lib().fgb_weight_quant_block128(_ptr(w), N, K, _ptr(w_q), _ptr(s_w), fmt, _stream())
    check("fgb_weight_quant_block128", st)
    return w_q, s_w


def _scale_fmt(s_w: torch.Tensor) -> int:
    if s_w.dtype == torch.float32:
        return SCALE_F32
    if s_w.dtype == torch.uint8:
        return SCALE_UE8M0
    raise ValueError("s_w must be float32 (scale_fmt 'float') or uint8 (scale_fmt 'ue8m0')")


def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return OUT_BF16
    if dtype == torch.float32:
        return OUT_F32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().fgb_gemm_workspace_bytes(M, N, K))


def gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
         out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = block-scaled (A_q . W_q^T) with 1x128 activation and 128x128 weight scales."""
    M, K = a_q.shape
    N = w_q.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    need = gemm_workspace_bytes(M, N, K)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=a_q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fgb_w8a8_block_gemm(_ptr(a_q), _row_ld(a_q), _ptr(s_a), s_a.stride(0), _ptr(w_q),
                                   _ptr(s_w), _scale_fmt(s_w), _ptr(out), _out_code(out.dtype),
                                   _row_ld(out), M, N, K, _ptr(workspace), ws_bytes, _stream())
    check("fgb_w8a8_block_gemm", st)
    return out


def grouped_gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
                 offsets: torch.Tensor, out_dtype=torch.bfloat16,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """MoE grouped GEMM: rows offsets[e]..offsets[e+1]-1 use expert e's weights and scales.

    offsets: int32 device tensor [E+1] (0, nondecreasing, ends at a_q.shape[0]).
    """
    total_M, K = a_q.shape
    E, N, _ = w_q.shape
    if offsets.dtype != torch.int32 or offsets.numel() != E + 1:
        raise ValueError("offsets must be an int32 tensor with E+1 entries")
    if out is None:
        out = torch.empty((total_M, N), dtype=out_dtype, device=a_q.device)
    st = lib().fgb_grouped_w8a8_block_gemm(_ptr(a_q), _row_ld(a_q), _ptr(s_a), s_a.stride(0), _ptr(w_q),
                                           _ptr(s_w), _scale_fmt(s_w), _ptr(offsets), E, total_M,
                                           _ptr(out), _out_code(out.dtype), _row_ld(out), N, K, None, 0,
                                           _stream())
    check("fgb_grouped_w8a8_block_gemm", st)
    return out


def check_offsets(offsets: torch.Tensor, total_M: int) -> int:
    """Check the grouped GEMM's expert offsets on the device (synchronizes): 0 when they start at
    0, never decrease and end at total_M, else 1 + the first index that breaks that."""
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous 1-D int32 tensor")
    result = torch.empty(1, dtype=torch.int32, device=offsets.device)
    st = lib().fgb_check_expert_offsets(_ptr(offsets), offsets.numel() - 1, total_M, _ptr(result), _stream())
    check("fgb_check_expert_offsets", st)
    return int(result.item())


def linear(x: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    """One fine-grained FP8 linear: dynamic activation quantization, then the block GEMM."""
    q, s_a = quantize(x)
    return gemm(q, s_a, w_q, s_w, out_dtype=out_dtype)


def fp8_encode(x: torch.Tensor, fmt: int = FP8_E4M3, saturate: bool = True) -> torch.Tensor:
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("fp8_encode expects a contiguous float32 tensor")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    check("fgb_fp8_encode", lib().fgb_fp8_encode(_ptr(x), _ptr(out), x.numel(), fmt, int(saturate), _stream()))
    return out


def fp8_decode(c: torch.Tensor, fmt: int = FP8_E4M3) -> torch.Tensor:
    if c.dtype != torch.uint8 or not c.is_contiguous():
        raise ValueError("fp8_decode expects a contiguous uint8 tensor")
    out = torch.empty(c.shape, dtype=torch.float32, device=c.device)
    check("fgb_fp8_decode", lib().fgb_fp8_decode(_ptr(c), _ptr(out), c.numel(), fmt, _stream()))
    return out


def selftest_quotients() -> tuple[int, int]:
    """Exhaustive device check of the quantizers' fast quotient (see include/fgb.h).

    Returns (pairs with differing E4M3 codes, pairs with differing float32 quotients).
    """
    counts = torch.zeros(2, dtype=torch.int64, device=torch.device("cuda", torch.cuda.current_device()))
    check("fgb_selftest_quotients", lib().fgb_selftest_quotients(_ptr(counts), _stream()))
    c = counts.cpu().tolist()
    return int(c[0]), int(c[1])
