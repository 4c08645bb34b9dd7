"""torch-tensor wrappers over the C-ABI (argument marshalling only).

Tensors must live on the current HIP device; outputs are allocated with torch and the calls
are enqueued on torch's current stream.  The C-ABI sees only base pointers and sizes, so it
cannot tell how large a buffer is: this layer checks every tensor's dtype, device, layout and
extent against the problem sizes before it calls the library, and raises ValueError on any
mismatch (a transposed or sliced weight would otherwise be read out of bounds by the kernels).
The library then validates what it can see (divisibility, leading dimensions, alignment) and
returns a status that is turned into FGBError (also a ValueError).
"""
from __future__ import annotations

import torch

from ._lib import (ACT_SCALE_TENSOR, ACT_SCALE_TOKEN, FP8_E4M3, FP8_E5M2, OUT_BF16, OUT_F32, SCALE_F32,
                   SCALE_UE8M0, W_SCALE_BLOCK128, W_SCALE_CHANNEL, check, lib)

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


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _matrix(t: torch.Tensor, name: str, dtype, rows: int | None = None, cols: int | None = None,
            min_cols: int | None = None) -> None:
    """t is a 2-D `dtype` tensor with unit inner stride, a row pitch of at least its width, and
    the given row count and width (or at least `min_cols` columns)."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.dim() == 2, f"{name} must be 2-D, got shape {tuple(t.shape)}")
    _need(t.stride(1) == 1 and t.stride(0) >= t.shape[1], f"{name} needs unit inner stride and row pitch >= width")
    if rows is not None:
        _need(t.shape[0] == rows, f"{name} must have {rows} rows, got {t.shape[0]}")
    if cols is not None:
        _need(t.shape[1] == cols, f"{name} must have {cols} columns, got {t.shape[1]}")
    if min_cols is not None:
        _need(t.shape[1] >= min_cols, f"{name} must have at least {min_cols} columns, got {t.shape[1]}")


def _dense(t: torch.Tensor, name: str, dtypes, shape: tuple) -> None:
    """t is a contiguous tensor of exactly `shape` with one of `dtypes`."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype in dtypes, f"{name} must be one of {dtypes}, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _on_device(*named) -> None:
    """Every tensor lives on the current HIP device (checked after the shapes, so that shape
    errors are reported without touching the device)."""
    cur = None
    for name, t in named:
        if t is None:
            continue
        _need(t.is_cuda, f"{name} must be on the GPU, got {t.device}")
        if cur is None:
            cur = torch.cuda.current_device()
        _need(t.device.index == cur, f"{name} is on {t.device}, the current device is cuda:{cur}")


def _blocks(n: int, what: str) -> int:
    _need(n % BLOCK == 0, f"{what} = {n} must be a multiple of {BLOCK}")
    return n // BLOCK


def quantize(x: torch.Tensor, out: tuple | None = None):
    """Dynamic per-token 1x128-group E4M3 quantization of bf16 activations.

    Returns (q uint8 [M, K], s_a float32 [K/128, ld_sa]) with ld_sa = M rounded up to 4;
    s_a[:, :M].t() is the logical [M, K/128] scale matrix.  `out` = (q, s_a) writes into given
    buffers: q uint8 [M, K] and s_a float32 [K/128, >= M], both with unit inner stride.
    """
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    KB = _blocks(K, "K")
    if out is None:
        _on_device(("x", x))
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s_a = torch.empty((KB, max(_ceil4(M), 4)), dtype=torch.float32, device=x.device)
    else:
        q, s_a = out
        _matrix(q, "q", torch.uint8, rows=M, cols=K)
        _matrix(s_a, "s_a", torch.float32, rows=KB, min_cols=M)
        _on_device(("x", x), ("q", q), ("s_a", s_a))
    st = lib().fgb_act_quant_group128(_ptr(x), M, K, _row_ld(x), _ptr(q), _row_ld(q), _ptr(s_a),
                                      s_a.stride(0), _stream())
    check("fgb_act_quant_group128", st)
    return q, s_a


_CODES = {"e4m3": FP8_E4M3, "e5m2": FP8_E5M2}


def _code(code: str) -> int:
    c = _CODES.get(code)
    _need(c is not None, "code must be 'e4m3' or 'e5m2'")
    return c


def quantize_weight(w: torch.Tensor, scale_fmt: str = "float", code: str = "e4m3"):
    """Per-128x128-block weight quantization of a dense bf16 [N, K] matrix.

    scale_fmt "float" -> s_w float32 [N/128, K/128]; "ue8m0" -> s_w uint8 UE8M0 codes.
    code "e4m3" (default) or "e5m2" (float32 scales amax/57344).
    """
    _need(isinstance(w, torch.Tensor) and w.dim() == 2, "quantize_weight expects a 2-D tensor")
    _dense(w, "w", (torch.bfloat16,), tuple(w.shape))
    N, K = w.shape
    NB, KB = _blocks(N, "N"), _blocks(K, "K")
    fmt = {"float": SCALE_F32, "ue8m0": SCALE_UE8M0}.get(scale_fmt)
    if fmt is None:
        raise ValueError("scale_fmt must be 'float' or 'ue8m0'")
    _on_device(("w", w))
    w_q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    sdt = torch.float32 if fmt == SCALE_F32 else torch.uint8
    s_w = torch.empty((max(NB, 1), max(KB, 1)), dtype=sdt, device=w.device)
    if code == "e4m3":
        st = lib().fgb_weight_quant_block128(_ptr(w), N, K, _ptr(w_q), _ptr(s_w), fmt, _stream())
        check("fgb_weight_quant_block128", st)
    else:
        st = lib().fgb_weight_quant_block128_ex(_ptr(w), N, K, _code(code), _ptr(w_q), _ptr(s_w), fmt, _stream())
        check("fgb_weight_quant_block128_ex", st)
    return w_q, s_w


def quantize_per_token(x: torch.Tensor, code: str = "e4m3", out: tuple | None = None):
    """Dynamic per-token quantization (FP8_DYNAMIC activations): one scale per row over the whole
    K.  Returns (q uint8 [M, K], s_a float32 [M])."""
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    _blocks(K, "K")
    if out is None:
        _on_device(("x", x))
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s_a = torch.empty((max(M, 1),), dtype=torch.float32, device=x.device)
    else:
        q, s_a = out
        _matrix(q, "q", torch.uint8, rows=M, cols=K)
        _dense(s_a, "s_a", (torch.float32,), (M,))
        _on_device(("x", x), ("q", q), ("s_a", s_a))
    st = lib().fgb_act_quant_per_token(_ptr(x), M, K, _row_ld(x), _code(code), _ptr(q), _row_ld(q), _ptr(s_a),
                                       _stream())
    check("fgb_act_quant_per_token", st)
    return q, s_a


def quantize_weight_per_channel(w: torch.Tensor, code: str = "e4m3"):
    """Per-output-channel weight quantization (FP8_DYNAMIC weights) of a dense bf16 [N, K]
    matrix.  Returns (w_q uint8 [N, K], s_w float32 [N])."""
    _need(isinstance(w, torch.Tensor) and w.dim() == 2, "expects a 2-D tensor")
    _dense(w, "w", (torch.bfloat16,), tuple(w.shape))
    N, K = w.shape
    _blocks(N, "N"), _blocks(K, "K")
    _on_device(("w", w))
    w_q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s_w = torch.empty((max(N, 1),), dtype=torch.float32, device=w.device)
    st = lib().fgb_weight_quant_per_channel(_ptr(w), N, K, _code(code), _ptr(w_q), _ptr(s_w), _stream())
    check("fgb_weight_quant_per_channel", st)
    return w_q, s_w


def quantize_static(x: torch.Tensor, scale: torch.Tensor, code: str = "e4m3", out: torch.Tensor | None = None):
    """Quantization with a given per-tensor scale (static activations): q = E(fl32(x / scale)).
    scale: float32 device tensor with one element (finite, > 0: not checked)."""
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    _blocks(K, "K")
    _dense(scale, "scale", (torch.float32,), tuple(scale.shape))
    _need(scale.numel() == 1, "scale must hold one value")
    if out is not None:
        _matrix(out, "out", torch.uint8, rows=M, cols=K)
    _on_device(("x", x), ("scale", scale), ("out", out))
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if out is None else out
    st = lib().fgb_act_quant_static(_ptr(x), M, K, _row_ld(x), _ptr(scale), _code(code), _ptr(q), _row_ld(q),
                                    _stream())
    check("fgb_act_quant_static", st)
    return q


def scaled_gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
                act_scale: str = "token", code: str = "e4m3", out_dtype=torch.bfloat16,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """GEMM with per-token (s_a float32 [M]) or per-tensor (s_a float32 [1]) activation scales and
    per-channel (s_w float32 [N]) or 128x128-block (s_w [N/128, K/128], float32 or UE8M0) weight
    scales; both operands in `code` ("e4m3" or "e5m2").  Decode sizes may need a workspace of
    gemm_workspace_bytes(M, N, K) bytes (allocated here when none is given)."""
    _matrix(a_q, "a_q", torch.uint8)
    M, K = a_q.shape
    KB = _blocks(K, "K")
    _need(isinstance(w_q, torch.Tensor) and w_q.dim() == 2, "w_q must be [N, K]")
    N = w_q.shape[0]
    NB = _blocks(N, "N")
    _dense(w_q, "w_q", (torch.uint8,), (N, K))
    if act_scale == "token":
        ak = ACT_SCALE_TOKEN
        _dense(s_a, "s_a", (torch.float32,), (M,))
    elif act_scale == "tensor":
        ak = ACT_SCALE_TENSOR
        _dense(s_a, "s_a", (torch.float32,), tuple(s_a.shape))
        _need(s_a.numel() == 1, "a per-tensor s_a holds one value")
    else:
        raise ValueError("act_scale must be 'token' or 'tensor'")
    if s_w.dim() == 1:
        wk = W_SCALE_CHANNEL
        _dense(s_w, "s_w", (torch.float32,), (N,))
    else:
        wk = W_SCALE_BLOCK128
        _dense(s_w, "s_w", (torch.float32, torch.uint8), (NB, KB))
    if out is not None:
        _need(out.dtype in (torch.bfloat16, torch.float32), "out must be bf16 or float32")
        _matrix(out, "out", out.dtype, rows=M, cols=N)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
    _on_device(("a_q", a_q), ("s_a", s_a), ("w_q", w_q), ("s_w", s_w), ("out", out), ("workspace", workspace))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    need = gemm_workspace_bytes(M, N, K)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=a_q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fgb_w8a8_scaled_gemm(_ptr(a_q), _row_ld(a_q), _ptr(s_a), ak, _ptr(w_q), _ptr(s_w), wk,
                                    _scale_fmt(s_w), _code(code), _ptr(out), _out_code(out.dtype), _row_ld(out),
                                    M, N, K, _ptr(workspace), ws_bytes, _stream())
    check("fgb_w8a8_scaled_gemm", st)
    return out


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


def _check_gemm_operands(a_q, s_a, w_q, s_w, out, E: int | None):
    """Shapes of the GEMM operands against M (rows of a_q), N, K (and E for grouped)."""
    _matrix(a_q, "a_q", torch.uint8)
    M, K = a_q.shape
    KB = _blocks(K, "K")
    _need(isinstance(w_q, torch.Tensor), "w_q must be a torch.Tensor")
    N = w_q.shape[-2] if w_q.dim() >= 2 else -1
    _need(w_q.dim() == (2 if E is None else 3), f"w_q must be {'[N, K]' if E is None else '[E, N, K]'}")
    NB = _blocks(N, "N")
    lead = () if E is None else (E,)
    _dense(w_q, "w_q", (torch.uint8,), lead + (N, K))
    _dense(s_w, "s_w", (torch.float32, torch.uint8), lead + (NB, KB))
    _matrix(s_a, "s_a", torch.float32, rows=KB, min_cols=M)
    if out is not None:
        _need(out.dtype in (torch.bfloat16, torch.float32), "out must be bf16 or float32")
        _matrix(out, "out", out.dtype, rows=M, cols=N)
    return M, N, K


def gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
         out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = block-scaled (A_q . W_q^T) with 1x128 activation and 128x128 weight scales.

    a_q uint8 [M, K] (unit inner stride); s_a float32 [K/128, >= M]; w_q uint8 [N, K] and s_w
    [N/128, K/128] (float32 or UE8M0 bytes), both contiguous; out [M, N] bf16 or float32.
    """
    M, N, K = _check_gemm_operands(a_q, s_a, w_q, s_w, out, None)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
    _on_device(("a_q", a_q), ("s_a", s_a), ("w_q", w_q), ("s_w", s_w), ("out", out), ("workspace", workspace))
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


def gemm_noalloc(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
                 out: torch.Tensor) -> torch.Tensor:
    """gemm() through the entry point that allocates nothing: the caller passes the output, and
    the decode calls that need a workspace use the library's own per-GPU scratch.  Calls that
    may overlap on one GPU must not be issued (they share that scratch)."""
    _need(out is not None, "gemm_noalloc writes into a given output tensor")
    M, N, K = _check_gemm_operands(a_q, s_a, w_q, s_w, out, None)
    _on_device(("a_q", a_q), ("s_a", s_a), ("w_q", w_q), ("s_w", s_w), ("out", out))
    st = lib().fgb_w8a8_block_gemm_noalloc(_ptr(a_q), _row_ld(a_q), _ptr(s_a), s_a.stride(0), _ptr(w_q),
                                           _ptr(s_w), _scale_fmt(s_w), _ptr(out), _out_code(out.dtype),
                                           _row_ld(out), M, N, K, _stream())
    check("fgb_w8a8_block_gemm_noalloc", st)
    return out


def grouped_gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
                 offsets: torch.Tensor, out_dtype=torch.bfloat16,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """MoE grouped GEMM: rows offsets[e]..offsets[e+1]-1 use expert e's weights and scales.

    w_q uint8 [E, N, K], s_w [E, N/128, K/128] contiguous; offsets: contiguous int32 device
    tensor [E+1] (0, nondecreasing, ends at a_q.shape[0]).
    """
    _need(isinstance(w_q, torch.Tensor) and w_q.dim() == 3, "w_q must be [E, N, K]")
    E = w_q.shape[0]
    total_M, N, K = _check_gemm_operands(a_q, s_a, w_q, s_w, out, E)
    _dense(offsets, "offsets", (torch.int32,), (E + 1,))
    _on_device(("a_q", a_q), ("s_a", s_a), ("w_q", w_q), ("s_w", s_w), ("offsets", offsets), ("out", out))
    if out is None:
        out = torch.empty((total_M, N), dtype=out_dtype, device=a_q.device)
    st = lib().fgb_grouped_w8a8_block_gemm(_ptr(a_q), _row_ld(a_q), _ptr(s_a), s_a.stride(0), _ptr(w_q),
                                           _ptr(s_w), _scale_fmt(s_w), _ptr(offsets), E, total_M,
                                           _ptr(out), _out_code(out.dtype), _row_ld(out), N, K, None, 0,
                                           _stream())
    check("fgb_grouped_w8a8_block_gemm", st)
    return out


def batched_gemm(a_q: torch.Tensor, s_a: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor,
                 counts: torch.Tensor, max_m: int, out_dtype=torch.bfloat16,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """MoE GEMM on the masked batched layout: expert e owns rows e*max_m .. e*max_m + counts[e]-1
    of a_q [E*max_m, K] (and of s_a, out); the rest of each slot is padding, left unwritten.

    counts: contiguous int32 device tensor [E] with 0 <= counts[e] <= max_m."""
    _need(isinstance(w_q, torch.Tensor) and w_q.dim() == 3, "w_q must be [E, N, K]")
    E = w_q.shape[0]
    rows, N, K = _check_gemm_operands(a_q, s_a, w_q, s_w, out, E)
    _need(int(max_m) >= 0 and rows == E * int(max_m), f"a_q must have E * max_m = {E * int(max_m)} rows")
    _dense(counts, "counts", (torch.int32,), (E,))
    _on_device(("a_q", a_q), ("s_a", s_a), ("w_q", w_q), ("s_w", s_w), ("counts", counts), ("out", out))
    if out is None:
        out = torch.empty((rows, N), dtype=out_dtype, device=a_q.device)
    st = lib().fgb_batched_w8a8_block_gemm(_ptr(a_q), _row_ld(a_q), _ptr(s_a), s_a.stride(0), _ptr(w_q),
                                           _ptr(s_w), _scale_fmt(s_w), _ptr(counts), E, int(max_m), _ptr(out),
                                           _out_code(out.dtype), _row_ld(out), N, K, _stream())
    check("fgb_batched_w8a8_block_gemm", st)
    return out


def check_offsets(offsets: torch.Tensor, total_M: int) -> int:
    """Check the grouped GEMM's expert offsets on the device (synchronizes): 0 when they start at
    0, never decrease and end at total_M, else 1 + the first index that breaks that."""
    _need(isinstance(offsets, torch.Tensor) and offsets.dim() == 1, "offsets must be 1-D")
    _dense(offsets, "offsets", (torch.int32,), tuple(offsets.shape))
    _on_device(("offsets", offsets))
    result = torch.empty(1, dtype=torch.int32, device=offsets.device)
    st = lib().fgb_check_expert_offsets(_ptr(offsets), offsets.numel() - 1, total_M, _ptr(result), _stream())
    check("fgb_check_expert_offsets", st)
    return int(result.item())


def gemm_fused_quant_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().fgb_gemm_fused_quant_workspace_bytes(M, N, K))


def gemm_fused_quant(x: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor, out_dtype=torch.bfloat16,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode-sized (M <= 64) fine-grained FP8 linear from bf16 activations in one call: the
    result of quantize() + gemm(), bit for bit.  A few tokens take one launch whose GEMM quantizes
    the activations itself; more tokens quantize into the workspace (allocated here when none of
    at least gemm_fused_quant_workspace_bytes(M, N, K) bytes is given)."""
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    KB = _blocks(K, "K")
    _need(M <= 64, "gemm_fused_quant is for M <= 64 (use quantize + gemm)")
    _need(isinstance(w_q, torch.Tensor) and w_q.dim() == 2, "w_q must be [N, K]")
    N = w_q.shape[0]
    NB = _blocks(N, "N")
    _dense(w_q, "w_q", (torch.uint8,), (N, K))
    _dense(s_w, "s_w", (torch.float32, torch.uint8), (NB, KB))
    if out is not None:
        _need(out.dtype in (torch.bfloat16, torch.float32), "out must be bf16 or float32")
        _matrix(out, "out", out.dtype, rows=M, cols=N)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
    _on_device(("x", x), ("w_q", w_q), ("s_w", s_w), ("out", out), ("workspace", workspace))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    need = gemm_fused_quant_workspace_bytes(M, N, K)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fgb_w8a8_block_gemm_fused_quant(_ptr(x), _row_ld(x), _ptr(w_q), _ptr(s_w), _scale_fmt(s_w), _ptr(out),
                                               _out_code(out.dtype), _row_ld(out), M, N, K, _ptr(workspace),
                                               ws_bytes, _stream())
    check("fgb_w8a8_block_gemm_fused_quant", st)
    return out


def linear(x: torch.Tensor, w_q: torch.Tensor, s_w: torch.Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    """One fine-grained FP8 linear: dynamic activation quantization, then the block GEMM."""
    q, s_a = quantize(x)
    return gemm(q, s_a, w_q, s_w, out_dtype=out_dtype)


def fp8_encode(x: torch.Tensor, fmt: int = FP8_E4M3, saturate: bool = True) -> torch.Tensor:
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("fp8_encode expects a contiguous float32 tensor")
    _on_device(("x", x))
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    check("fgb_fp8_encode", lib().fgb_fp8_encode(_ptr(x), _ptr(out), x.numel(), fmt, int(saturate), _stream()))
    return out


def fp8_decode(c: torch.Tensor, fmt: int = FP8_E4M3) -> torch.Tensor:
    if c.dtype != torch.uint8 or not c.is_contiguous():
        raise ValueError("fp8_decode expects a contiguous uint8 tensor")
    _on_device(("c", c))
    out = torch.empty(c.shape, dtype=torch.float32, device=c.device)
    check("fgb_fp8_decode", lib().fgb_fp8_decode(_ptr(c), _ptr(out), c.numel(), fmt, _stream()))
    return out


def selftest_quotients() -> tuple[int, int, int]:
    """Exhaustive device check of the quantizers' fast quotient (see include/fgb.h).

    Returns (pairs with differing E4M3 codes, pairs with differing float32 quotients, pairs with
    differing quotients of magnitude >= 2^-13).
    """
    counts = torch.zeros(3, dtype=torch.int64, device=torch.device("cuda", torch.cuda.current_device()))
    check("fgb_selftest_quotients", lib().fgb_selftest_quotients(_ptr(counts), _stream()))
    c = counts.cpu().tolist()
    return int(c[0]), int(c[1]), int(c[2])
