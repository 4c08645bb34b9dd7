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
from oracle import blockquant, gemm, schemes
from tests.gemm_helpers import bf16_tensor_to_f64, check_t2

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pick(rng, M, N, nrows=64, nblocks=8):
    """Token rows (always the first and the last, and both sides of the first 256-row tile edge)
    and the columns of whole 128-row weight blocks (always the first and the last block, and both
    sides of the first 256-column tile edge)."""
    if M <= nrows:
        rows = np.arange(M)
    else:
        fixed = [0, M - 1] + ([255, 256] if M > 256 else [])
        rows = np.unique(np.concatenate([fixed, rng.choice(M, nrows - len(fixed), replace=False)]))
    nb = N // 128
    fixed = [0, nb - 1] + ([1, 2] if nb > 2 and nblocks >= 4 else [])
    extra = max(0, min(nblocks, nb) - len(fixed))
    blocks = np.unique(np.concatenate([fixed, rng.choice(nb, extra, replace=False)]).astype(np.int64))
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


def _check_tiles_in_place(dev, M, N, K, fmt, seed):
    """Every output tile at full size, without the oracle: a row's sums do not depend on where it
    sits (same K-block order, same lane inside its 16-row MFMA tile), so permuting the weight
    rows by whole 128-row blocks (with their scales) must permute the output columns, and
    permuting the activation rows by groups of 16 (with their scales) must permute the output
    rows, bit for bit.  A tile computed from the wrong operands or stored to the wrong place
    (the persistent walk, the per-XCD order, the split between 256x256 and 256x128 tiles)
    breaks the equality."""
    x = workloads.device_bf16((M, K), seed, dev)
    w = workloads.device_bf16((N, K), seed + 1, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w, "float" if fmt == "f32" else "ue8m0")
    q, sa = fgb.quantize(x)
    del x, w
    y = fgb.gemm(q, sa, wq, sw)
    rng = np.random.default_rng(seed)
    pb = _idx(rng.permutation(N // 128), dev)
    y_w = fgb.gemm(q, sa, wq.view(N // 128, 128, K)[pb].reshape(N, K).contiguous(), sw[pb].contiguous())
    pg = rng.permutation(M // 16)
    pr = _idx((pg[:, None] * 16 + np.arange(16)[None, :]).reshape(-1), dev)
    sa_p = torch.zeros_like(sa)
    sa_p[:, :M] = sa[:, pr]
    y_a = fgb.gemm(q[pr].contiguous(), sa_p, wq, sw)
    torch.cuda.synchronize()
    expect_w = y.view(M, N // 128, 128)[:, pb].reshape(M, N)
    assert torch.equal(y_w.view(torch.int16), expect_w.view(torch.int16))
    assert torch.equal(y_a.view(torch.int16), y[pr].view(torch.int16))


@pytest.mark.parametrize("name,N,K", workloads.DEEPSEEK_V3_LINEARS, ids=[s[0] for s in workloads.DEEPSEEK_V3_LINEARS])
def test_deepseek_v3_prefill_m8192_every_tile_in_place(dev, name, N, K):
    _check_tiles_in_place(dev, workloads.DEEPSEEK_V3_PREFILL_M, N, K, "ue8m0", seed=sum(map(ord, name)) + 300)


@pytest.mark.parametrize("name,N,K", workloads.LLAMA3_8B_LINEARS, ids=[s[0] for s in workloads.LLAMA3_8B_LINEARS])
def test_llama3_8b_prefill_m4096_every_tile_in_place(dev, name, N, K):
    _check_tiles_in_place(dev, workloads.LLAMA3_8B_PREFILL_M, N, K, "f32", seed=sum(map(ord, name)) + 350)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_moe_grouped_full_every_tile_in_place(dev, proj):
    """The 32-expert grouped GEMM at full size: permuting every expert's weight rows by the same
    whole 128-row blocks (with their scales) must permute the output columns bit for bit."""
    cfg = workloads.MOE
    E = cfg["E"]
    N, K = cfg[proj]
    _, offsets, _ = workloads.moe_routing(cfg["tokens"], E, cfg["topk"], cfg["zipf"])
    T = int(offsets[-1])
    seed = 600 if proj == "gate_up" else 650
    x = workloads.device_bf16((T, K), seed, dev)
    w = workloads.device_bf16((E * N, K), seed + 1, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    q, sa = fgb.quantize(x)
    del x, w
    off = torch.from_numpy(offsets).to(dev)
    wq3, sw3 = wq.view(E, N, K), sw.view(E, N // 128, K // 128)
    y = fgb.grouped_gemm(q, sa, wq3, sw3, off)
    pb = _idx(np.random.default_rng(seed).permutation(N // 128), dev)
    y_w = fgb.grouped_gemm(q, sa, wq3.view(E, N // 128, 128, K)[:, pb].reshape(E, N, K).contiguous(),
                           sw3[:, pb].contiguous(), off)
    torch.cuda.synchronize()
    assert torch.equal(y_w.view(torch.int16), y.view(T, N // 128, 128)[:, pb].reshape(T, N).view(torch.int16))


@pytest.mark.parametrize("name,N,K", workloads.DECODE_SHAPES, ids=[s[0] for s in workloads.DECODE_SHAPES])
def test_decode_full_shapes_every_tile_in_place(dev, name, N, K):
    """The decode kernels at every full decode shape (M = 1, 8, 32, 64: register, per-wave ring,
    2/4/8-wave shared-ring kernels, K slices and their reduction): the permutation checks of
    the prefill shapes, columns always, rows by 16-row groups where M has more than one."""
    seed = sum(map(ord, name)) + 800
    w = workloads.device_bf16((N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    del w
    rng = np.random.default_rng(seed)
    pb = _idx(rng.permutation(N // 128), dev)
    wq_p = wq.view(N // 128, 128, K)[pb].reshape(N, K).contiguous()
    sw_p = sw[pb].contiguous()
    for M in (1, 8, 32, 64):
        x = workloads.device_bf16((M, K), seed + M, dev)
        q, sa = fgb.quantize(x)
        y = fgb.gemm(q, sa, wq, sw)
        y_w = fgb.gemm(q, sa, wq_p, sw_p)
        torch.cuda.synchronize()
        assert torch.equal(y_w.view(torch.int16), y.view(M, N // 128, 128)[:, pb].reshape(M, N).view(torch.int16)), M
        if M >= 32:
            pg = rng.permutation(M // 16)
            pr = _idx((pg[:, None] * 16 + np.arange(16)[None, :]).reshape(-1), dev)
            sa_p = torch.zeros_like(sa)
            sa_p[:, :M] = sa[:, pr]
            y_a = fgb.gemm(q[pr].contiguous(), sa_p, wq, sw)
            torch.cuda.synchronize()
            assert torch.equal(y_a.view(torch.int16), y[pr].view(torch.int16)), M


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
    """32 experts, 4096 tokens routed top-8 with Zipf(1.1) expert popularity (32768 rows); in
    every expert its first and last rows, both sides of its first 256-row tile edge and two random
    rows, on two sampled weight blocks (the last always)."""
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
    rng = np.random.default_rng(seed)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        rows = [r0, r1 - 1] + [r for r in (r0 + 255, r0 + 256) if r < r1]
        rows = np.unique(np.concatenate([rows, rng.integers(r0, r1, size=2)]))
        _, cols = _pick(rng, 1, N, nblocks=2)
        aq, sa_o = blockquant.act_quant(_bits(x[_idx(rows, dev)]))
        wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(e * N + cols, dev)]), "f32")
        yref = gemm.gemm_ref(aq, sa_o, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)


# ------------------------------------------------------------------------------------------
# the other paths at full size, in the launch configuration bench.py times
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,N,K", [workloads.LLAMA3_8B_LINEARS[2], workloads.LLAMA3_8B_LINEARS[3]],
                         ids=["gate_up", "down"])
def test_fp8_dynamic_llama3_8b_m4096(dev, name, N, K):
    """Per-token activations, per-channel weights (E4M3); each sampled row and weight row is
    quantized independently of the others, so the oracle quantizes exactly the sample."""
    M = workloads.LLAMA3_8B_PREFILL_M
    seed = sum(map(ord, name)) + 600
    x = workloads.device_bf16((M, K), seed, dev)
    w = workloads.device_bf16((N, K), seed + 1, dev, outliers=False, std=0.02)
    q, sa = fgb.quantize_per_token(x)
    wq, sw = fgb.quantize_weight_per_channel(w)
    y = fgb.scaled_gemm(q, sa, wq, sw, act_scale="token")
    torch.cuda.synchronize()
    rows, cols = _pick(np.random.default_rng(seed), M, N)
    aq, sa_o = schemes.token_quant(_bits(x[_idx(rows, dev)]))
    wq_s, sw_s = schemes.channel_weight_quant(_bits(w[_idx(cols, dev)]))
    yref = schemes.scaled_gemm_ref(aq, sa_o, wq_s, sw_s, act="token", weight="channel")
    check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)


def test_static_e5m2_llama3_8b_gate_up(dev):
    """Static per-tensor activation scale with E5M2 codes and E5M2 128x128 weight blocks."""
    M, (name, N, K) = workloads.LLAMA3_8B_PREFILL_M, workloads.LLAMA3_8B_LINEARS[2]
    x = workloads.device_bf16((M, K), 700, dev)
    w = workloads.device_bf16((N, K), 701, dev, outliers=False, std=0.02)
    s = np.float32(float(x.float().abs().max()) / 57344.0)
    q = fgb.quantize_static(x, torch.tensor([s], device=dev), "e5m2")
    wq, sw = fgb.quantize_weight(w, "float", code="e5m2")
    y = fgb.scaled_gemm(q, torch.tensor([s], device=dev), wq, sw, act_scale="tensor", code="e5m2")
    torch.cuda.synchronize()
    rows, cols = _pick(np.random.default_rng(700), M, N)
    aq = schemes.static_quant(_bits(x[_idx(rows, dev)]), s, "e5m2")
    wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(cols, dev)]), "f32", code="e5m2")
    yref = schemes.scaled_gemm_ref(aq, s, wq_s, sw_s, act="tensor", weight="block", a_code="e5m2", w_code="e5m2")
    check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)


@pytest.mark.parametrize("name,N,K", workloads.DECODE_SHAPES, ids=[s[0] for s in workloads.DECODE_SHAPES])
def test_fused_quant_decode_full_shapes(dev, name, N, K):
    """The fused-quantization decode GEMM at every decode batch size and the full weight shape."""
    seed = sum(map(ord, name)) + 800
    w = workloads.device_bf16((N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    _, cols = _pick(np.random.default_rng(seed), 1, N)
    wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(cols, dev)]), "f32")
    for M in workloads.DECODE_MS:
        x = workloads.device_bf16((M, K), seed + M, dev)
        y = fgb.gemm_fused_quant(x, wq, sw)
        torch.cuda.synchronize()
        aq, sa = blockquant.act_quant(_bits(x))
        yref = gemm.gemm_ref(aq, sa, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[:, _idx(cols, dev)]), yref)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("tokens", [1, 8, 64])
def test_moe_decode_shaped_full(dev, proj, tokens):
    """32 experts at the full expert shapes, top-8 Zipf routing of a few tokens: the grouped
    layout (8 or 64 rows in all) or, for 64 tokens, the batched layout with 64-row slots; every
    routed row against the oracle on sampled weight columns."""
    cfg = workloads.MOE
    E = cfg["E"]
    N, K = cfg[proj]
    _, offsets, counts = workloads.moe_routing(tokens=tokens, key=(0, 9, tokens, 1))
    seed = 900 + tokens + (0 if proj == "gate_up" else 50)
    w = workloads.device_bf16((E * N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    wq3, sw3 = wq.view(E, N, K), sw.view(E, N // 128, K // 128)
    if tokens <= 8:
        T = int(offsets[-1])
        x = workloads.device_bf16((T, K), seed + 1, dev)
        q, sa = fgb.quantize(x)
        y = fgb.grouped_gemm(q, sa, wq3, sw3, torch.from_numpy(offsets).to(dev))
        spans = [(e, offsets[e], offsets[e + 1]) for e in range(E)]
    else:
        slot = 64
        cnt = np.minimum(counts, slot).astype(np.int32)
        x = workloads.device_bf16((E * slot, K), seed + 1, dev)
        q, sa = fgb.quantize(x)
        y = fgb.batched_gemm(q, sa, wq3, sw3, torch.from_numpy(cnt).to(dev), slot)
        spans = [(e, e * slot, e * slot + cnt[e]) for e in range(E)]
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for e, r0, r1 in spans:
        if r1 <= r0:
            continue
        rows = np.arange(r0, r1)
        _, cols = _pick(rng, 1, N, nblocks=2)
        aq, sa_o = blockquant.act_quant(_bits(x[_idx(rows, dev)]))
        wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(e * N + cols, dev)]), "f32")
        yref = gemm.gemm_ref(aq, sa_o, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)



@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("tokens", [8, 64])
def test_moe_decode_shaped_full_every_tile_in_place(dev, proj, tokens):
    """The decode-shaped MoE calls at the full expert shapes (grouped 64 rows, batched 64-row
    slots): permuting every expert's weight rows by the same whole 128-row blocks (with their
    scales) must permute the output columns bit for bit."""
    cfg = workloads.MOE
    E = cfg["E"]
    N, K = cfg[proj]
    _, offsets, counts = workloads.moe_routing(tokens=tokens, key=(0, 9, tokens, 1))
    seed = 950 + tokens + (0 if proj == "gate_up" else 50)
    w = workloads.device_bf16((E * N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    del w
    wq3, sw3 = wq.view(E, N, K), sw.view(E, N // 128, K // 128)
    pb = _idx(np.random.default_rng(seed).permutation(N // 128), dev)
    wq_p = wq3.view(E, N // 128, 128, K)[:, pb].reshape(E, N, K).contiguous()
    sw_p = sw3[:, pb].contiguous()
    if tokens == 8:
        T = int(offsets[-1])
        q, sa = fgb.quantize(workloads.device_bf16((T, K), seed + 1, dev))
        off = torch.from_numpy(offsets).to(dev)
        y = fgb.grouped_gemm(q, sa, wq3, sw3, off)
        y_w = fgb.grouped_gemm(q, sa, wq_p, sw_p, off)
        valid = torch.ones(T, dtype=torch.bool, device=dev)
    else:
        slot = 64
        cnt = torch.from_numpy(np.minimum(counts, slot).astype(np.int32)).to(dev)
        T = E * slot
        q, sa = fgb.quantize(workloads.device_bf16((T, K), seed + 1, dev))
        y = fgb.batched_gemm(q, sa, wq3, sw3, cnt, slot)
        y_w = fgb.batched_gemm(q, sa, wq_p, sw_p, cnt, slot)
        valid = (torch.arange(slot, device=dev)[None, :] < cnt[:, None]).reshape(-1)
    torch.cuda.synchronize()
    expect = y.view(T, N // 128, 128)[:, pb].reshape(T, N)
    assert torch.equal(y_w[valid].view(torch.int16), expect[valid].view(torch.int16))
