"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Inputs are drawn on the device (workloads.device_bf16, seeded); the library quantizes them and
runs the block GEMM with bf16 output, exactly as in bench.py.  The oracle cannot afford these
sizes whole, but quantization is independent per token row and per 128x128 weight block, so for
a sample of token rows and of 128-row weight blocks the oracle quantizes the very bf16 bytes the
device holds (copied back) and computes those outputs exactly; they must meet the bf16 bound
|y16 - y_ref| <= 2e-3 max|y_ref| + 1 bf16 ulp (max over the sample).
"""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t2

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pick(rng, M, N, nrows=16, nblocks=2):
    """Token rows (always the first and the last) and the columns of whole 128-row weight blocks
    (always the last block)."""
    if M <= nrows:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nrows - 2, replace=False)]))
    nb = N // 128
    blocks = np.unique(np.concatenate([[nb - 1], rng.choice(nb, nblocks - 1, replace=False)]))
    cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    return rows, cols


def _idx(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev)


def _check_dense(dev, M, N, K, fmt, seed):
    x = workloads.device_bf16((M, K), seed, dev)
    w = workloads.device_bf16((N, K), seed + 1, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w, "float" if fmt == "f32" else "ue8m0")
    y = fgb.linear(x, wq, sw)
    torch.cuda.synchronize()
    rows, cols = _pick(np.random.default_rng(seed), M, N)
    aq, sa = blockquant.act_quant(_bits(x[_idx(rows, dev)]))
    wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(cols, dev)]), fmt)
    yref = gemm.gemm_ref(aq, sa, wq_s, sw_s, fmt)
    got = bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)])
    check_t2(got, yref)


@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_8B_LINEARS, ids=[s[0] for s in workloads.LLAMA3_8B_LINEARS])
def test_llama3_8b_prefill_m4096(dev, name, N, K):
    _check_dense(dev, workloads.LLAMA3_8B_PREFILL_M, N, K, "f32", seed=sum(map(ord, name)) + 100)


@pytest.mark.parametrize("name,N,K", workloads.DEEPSEEK_V3_LINEARS, ids=[s[0] for s in workloads.DEEPSEEK_V3_LINEARS])
def test_deepseek_v3_prefill_m8192_ue8m0(dev, name, N, K):
    _check_dense(dev, workloads.DEEPSEEK_V3_PREFILL_M, N, K, "ue8m0", seed=sum(map(ord, name)) + 200)


@pytest.mark.parametrize("name,N,K", workloads.DECODE_SHAPES, ids=[s[0] for s in workloads.DECODE_SHAPES])
def test_decode_full_shapes(dev, name, N, K):
    """Every decode batch size at the full weight shape; all M rows are checked."""
    seed = sum(map(ord, name)) + 300
    w = workloads.device_bf16((N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    _, cols = _pick(np.random.default_rng(seed), 1, N)
    wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(cols, dev)]), "f32")
    for M in workloads.DECODE_MS:
        x = workloads.device_bf16((M, K), seed + M, dev)
        y = fgb.linear(x, wq, sw)
        torch.cuda.synchronize()
        aq, sa = blockquant.act_quant(_bits(x))
        yref = gemm.gemm_ref(aq, sa, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[:, _idx(cols, dev)]), yref)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_moe_grouped_full(dev, proj):
    """32 experts, 4096 tokens routed top-8 with Zipf(1.1) expert popularity (32768 rows); the
    first and last rows of six experts (the most and least loaded among them) are checked."""
    cfg = workloads.MOE
    E = cfg["E"]
    N, K = cfg[proj]
    token_of_row, offsets, counts = workloads.moe_routing(cfg["tokens"], E, cfg["topk"], cfg["zipf"])
    seed = 400 if proj == "gate_up" else 500
    xt = workloads.device_bf16((cfg["tokens"], K), seed, dev)
    x = xt[_idx(token_of_row, dev)].contiguous()
    w = workloads.device_bf16((E * N, K), seed + 1, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    q, sa = fgb.quantize(x)
    off = torch.from_numpy(offsets).to(dev)
    y = fgb.grouped_gemm(q, sa, wq.view(E, N, K), sw.view(E, N // 128, K // 128), off)
    torch.cuda.synchronize()
    order = np.argsort(counts)
    experts = np.unique(np.concatenate([order[:2], order[-2:], order[E // 2 - 1:E // 2 + 1]]))
    rng = np.random.default_rng(seed)
    for e in experts:
        if counts[e] == 0:
            continue
        rows = np.unique([offsets[e], offsets[e + 1] - 1])
        _, cols = _pick(rng, 1, N)
        aq, sa_o = blockquant.act_quant(_bits(x[_idx(rows, dev)]))
        wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(e * N + cols, dev)]), "f32")
        yref = gemm.gemm_ref(aq, sa_o, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)
