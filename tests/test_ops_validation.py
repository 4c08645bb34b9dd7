"""The Python binding checks every tensor against the problem sizes before calling the library
(the C-ABI sees only base pointers).  These run on the CPU: mismatched tensors must raise
ValueError before anything reaches the library, and correctly shaped host tensors must be
refused because they are not on the GPU."""
import pytest
import torch

import fine_grained_block_amd as fgb
from fine_grained_block_amd import _lib


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    """Any call into the library fails the test: validation must stop every case first."""
    def boom():
        raise AssertionError("the library was called")
    monkeypatch.setattr(_lib, "lib", boom)
    monkeypatch.setattr(fgb.ops, "lib", boom)


def _ops(M=96, N=256, K=512, E=None):
    lead = () if E is None else (E,)
    a_q = torch.zeros((M, K), dtype=torch.uint8)
    s_a = torch.zeros((K // 128, (M + 3) // 4 * 4), dtype=torch.float32)
    w_q = torch.zeros(lead + (N, K), dtype=torch.uint8)
    s_w = torch.zeros(lead + (N // 128, K // 128), dtype=torch.float32)
    return a_q, s_a, w_q, s_w


def test_gemm_host_tensors_are_refused():
    a_q, s_a, w_q, s_w = _ops()
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.gemm(a_q, s_a, w_q, s_w)


@pytest.mark.parametrize("case", [
    "w_transposed", "w_sliced_rows", "w_wrong_k", "sw_shape", "sw_dtype", "sa_rows", "sa_too_few_tokens",
    "sa_strided", "a_dtype", "a_not_unit_stride", "out_shape", "out_dtype", "k_not_block",
])
def test_gemm_shape_mismatch(case):
    a_q, s_a, w_q, s_w = _ops()
    out = None
    if case == "w_transposed":
        w_q = torch.zeros((512, 256), dtype=torch.uint8).t()
    elif case == "w_sliced_rows":
        w_q = torch.zeros((256, 1024), dtype=torch.uint8)[:, :512]
    elif case == "w_wrong_k":
        w_q = torch.zeros((256, 384), dtype=torch.uint8)
    elif case == "sw_shape":
        s_w = torch.zeros((2, 3), dtype=torch.float32)
    elif case == "sw_dtype":
        s_w = s_w.to(torch.float64)
    elif case == "sa_rows":
        s_a = torch.zeros((3, 96), dtype=torch.float32)
    elif case == "sa_too_few_tokens":
        s_a = torch.zeros((4, 64), dtype=torch.float32)
    elif case == "sa_strided":
        s_a = torch.zeros((96, 4), dtype=torch.float32).t()
    elif case == "a_dtype":
        a_q = a_q.to(torch.int8)
    elif case == "a_not_unit_stride":
        a_q = torch.zeros((96, 1024), dtype=torch.uint8)[:, ::2]
    elif case == "out_shape":
        out = torch.zeros((96, 128), dtype=torch.bfloat16)
    elif case == "out_dtype":
        out = torch.zeros((96, 256), dtype=torch.float16)
    elif case == "k_not_block":
        a_q = torch.zeros((96, 500), dtype=torch.uint8)
    with pytest.raises(ValueError) as ei:
        fgb.gemm(a_q, s_a, w_q, s_w, out=out)
    assert "on the GPU" not in str(ei.value)


@pytest.mark.parametrize("case", ["offsets_len", "offsets_dtype", "w_2d", "sw_experts", "w_noncontig"])
def test_grouped_shape_mismatch(case):
    a_q, s_a, w_q, s_w = _ops(E=4)
    offsets = torch.zeros(5, dtype=torch.int32)
    if case == "offsets_len":
        offsets = torch.zeros(4, dtype=torch.int32)
    elif case == "offsets_dtype":
        offsets = offsets.to(torch.int64)
    elif case == "w_2d":
        w_q = w_q[0]
    elif case == "sw_experts":
        s_w = s_w[:3]
    elif case == "w_noncontig":
        w_q = torch.zeros((4, 512, 512), dtype=torch.uint8)[:, ::2]
    with pytest.raises(ValueError) as ei:
        fgb.grouped_gemm(a_q, s_a, w_q, s_w, offsets)
    assert "on the GPU" not in str(ei.value)


def test_grouped_host_tensors_are_refused():
    a_q, s_a, w_q, s_w = _ops(E=4)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.grouped_gemm(a_q, s_a, w_q, s_w, torch.zeros(5, dtype=torch.int32))


@pytest.mark.parametrize("case", ["q_shape", "sa_rows", "sa_tokens", "x_dtype", "k_not_block"])
def test_quantize_mismatch(case):
    x = torch.zeros((10, 256), dtype=torch.bfloat16)
    q = torch.zeros((10, 256), dtype=torch.uint8)
    s_a = torch.zeros((2, 12), dtype=torch.float32)
    if case == "q_shape":
        q = torch.zeros((10, 128), dtype=torch.uint8)
    elif case == "sa_rows":
        s_a = torch.zeros((1, 12), dtype=torch.float32)
    elif case == "sa_tokens":
        s_a = torch.zeros((2, 8), dtype=torch.float32)
    elif case == "x_dtype":
        x = x.float()
    elif case == "k_not_block":
        x = torch.zeros((10, 200), dtype=torch.bfloat16)
    with pytest.raises(ValueError) as ei:
        fgb.quantize(x, out=(q, s_a))
    assert "on the GPU" not in str(ei.value)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.quantize(torch.zeros((10, 256), dtype=torch.bfloat16))


def test_quantize_weight_mismatch():
    with pytest.raises(ValueError):
        fgb.quantize_weight(torch.zeros((256, 256), dtype=torch.bfloat16).t()[:, :128])
    with pytest.raises(ValueError):
        fgb.quantize_weight(torch.zeros((200, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.quantize_weight(torch.zeros((256, 256), dtype=torch.bfloat16))


@pytest.mark.parametrize("case", ["rows_not_e_slots", "counts_len", "counts_dtype", "w_2d"])
def test_batched_shape_mismatch(case):
    a_q, s_a, w_q, s_w = _ops(M=64, E=4)   # 4 slots of 16 rows
    counts = torch.zeros(4, dtype=torch.int32)
    max_m = 16
    if case == "rows_not_e_slots":
        max_m = 20
    elif case == "counts_len":
        counts = torch.zeros(3, dtype=torch.int32)
    elif case == "counts_dtype":
        counts = counts.to(torch.int64)
    elif case == "w_2d":
        w_q = w_q[0]
    with pytest.raises(ValueError) as ei:
        fgb.batched_gemm(a_q, s_a, w_q, s_w, counts, max_m)
    assert "on the GPU" not in str(ei.value)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.batched_gemm(*_ops(M=64, E=4), torch.zeros(4, dtype=torch.int32), 16)


@pytest.mark.parametrize("case", ["token_len", "tensor_two", "channel_len", "block_shape", "act_kind", "w_shape",
                                  "out_shape"])
def test_scaled_gemm_shape_mismatch(case):
    M, N, K = 24, 256, 512
    a_q = torch.zeros((M, K), dtype=torch.uint8)
    w_q = torch.zeros((N, K), dtype=torch.uint8)
    s_a = torch.zeros(M, dtype=torch.float32)
    s_w = torch.zeros(N, dtype=torch.float32)
    act, out = "token", None
    if case == "token_len":
        s_a = torch.zeros(M + 1, dtype=torch.float32)
    elif case == "tensor_two":
        act, s_a = "tensor", torch.zeros(2, dtype=torch.float32)
    elif case == "channel_len":
        s_w = torch.zeros(N - 1, dtype=torch.float32)
    elif case == "block_shape":
        s_w = torch.zeros((2, 3), dtype=torch.float32)
    elif case == "act_kind":
        act = "group"
    elif case == "w_shape":
        w_q = torch.zeros((N, K + 128), dtype=torch.uint8)
    elif case == "out_shape":
        out = torch.zeros((M, N + 1), dtype=torch.float32)
    with pytest.raises(ValueError) as ei:
        fgb.scaled_gemm(a_q, s_a, w_q, s_w, act_scale=act, out=out)
    assert "on the GPU" not in str(ei.value)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.scaled_gemm(torch.zeros((M, K), dtype=torch.uint8), torch.zeros(M, dtype=torch.float32),
                        torch.zeros((N, K), dtype=torch.uint8), torch.zeros(N, dtype=torch.float32))


@pytest.mark.parametrize("case", ["m_too_large", "x_dtype", "w_shape", "sw_shape", "out_shape"])
def test_fused_quant_shape_mismatch(case):
    M, N, K = 8, 256, 512
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    w_q = torch.zeros((N, K), dtype=torch.uint8)
    s_w = torch.zeros((N // 128, K // 128), dtype=torch.float32)
    out = None
    if case == "m_too_large":
        x = torch.zeros((65, K), dtype=torch.bfloat16)
    elif case == "x_dtype":
        x = x.float()
    elif case == "w_shape":
        w_q = torch.zeros((N, K - 128), dtype=torch.uint8)
    elif case == "sw_shape":
        s_w = torch.zeros((N // 128, K // 128 + 1), dtype=torch.float32)
    elif case == "out_shape":
        out = torch.zeros((M + 1, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError) as ei:
        fgb.gemm_fused_quant(x, w_q, s_w, out=out)
    assert "on the GPU" not in str(ei.value)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.gemm_fused_quant(torch.zeros((M, K), dtype=torch.bfloat16), torch.zeros((N, K), dtype=torch.uint8),
                             torch.zeros((N // 128, K // 128), dtype=torch.float32))


def test_noalloc_and_scheme_quantizers_mismatch():
    a_q, s_a, w_q, s_w = _ops()
    with pytest.raises(ValueError):
        fgb.gemm_noalloc(a_q, s_a, w_q, s_w, None)
    with pytest.raises(ValueError):
        fgb.gemm_noalloc(a_q, s_a, w_q, s_w, torch.zeros((96, 128), dtype=torch.bfloat16))
    x = torch.zeros((10, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fgb.quantize_per_token(x, out=(torch.zeros((10, 256), dtype=torch.uint8), torch.zeros(9, dtype=torch.float32)))
    with pytest.raises(ValueError):
        fgb.quantize_static(x, torch.zeros(2, dtype=torch.float32))
    with pytest.raises(ValueError):
        fgb.quantize_static(x, torch.ones(1, dtype=torch.float32), out=torch.zeros((10, 128), dtype=torch.uint8))
    with pytest.raises(ValueError):
        fgb.quantize_weight_per_channel(torch.zeros((200, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.quantize_per_token(x)
    with pytest.raises(ValueError, match="on the GPU"):
        fgb.quantize_static(x, torch.ones(1, dtype=torch.float32))
