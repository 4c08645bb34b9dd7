"""GPU parity: grouped (MoE) block-scaled GEMM against the oracle's per-expert loop."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, sa_device

pytestmark = pytest.mark.gpu


def _experts(E, N, K, key, fmt="f32"):
    wq = np.empty((E, N, K), np.uint8)
    sw = np.empty((E, N // 128, K // 128), np.float32 if fmt == "f32" else np.uint8)
    for e in range(E):
        wq[e], sw[e] = blockquant.weight_quant(workloads.weights(N, K, key=(key, 30, 1, e)), fmt)
    return wq, sw


def _run(aq, sa, wq, sw, offsets, dev, dt):
    y = fgb.grouped_gemm(torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq).to(dev),
                         torch.from_numpy(sw).to(dev), torch.from_numpy(offsets.astype(np.int32)).to(dev),
                         out_dtype=dt)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("counts", [[7, 0, 300, 130], [0, 0, 257, 0], [129], [1, 1, 1, 1, 1, 1, 1, 1], [0, 513]])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("K", [512, 4096])  # K >= 4096 takes the 256 x 256 tiles
def test_grouped_parity(dev, counts, fmt, K):
    E, N = len(counts), 256
    offsets = workloads.offsets_from_counts(counts)
    T = int(offsets[-1])
    x = workloads.activations(T, K, key=(0, 31, 0, T))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, key=sum(counts), fmt=fmt)
    yref = gemm.grouped_ref(aq, sa, wq, sw, offsets, fmt)
    y32 = _run(aq, sa, wq, sw, offsets, dev, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run(aq, sa, wq, sw, offsets, dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)


@pytest.mark.parametrize("K", [512, 1024])  # 256 x 128 and 256 x 256 tiles
def test_grouped_many_experts(dev, K):
    """130 experts: the tile-row counts and the expert lookup run over three 63-expert wave
    passes; empty experts sit at the pass edges and the last pass holds rows."""
    rng = np.random.default_rng(130)
    counts = rng.integers(0, 160, 130)
    counts[[0, 62, 63, 64, 125, 126]] = 0
    counts[[61, 127, 129]] = [257, 1, 300]
    offsets = workloads.offsets_from_counts(counts)
    T, E, N = int(offsets[-1]), 130, 256
    x = workloads.activations(T, K, key=(0, 34, 0, T))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, key=34)
    yref = gemm.grouped_ref(aq, sa, wq, sw, offsets)
    y16 = _run(aq, sa, wq, sw, offsets, dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("K", [1024, 2048, 7168])
def test_grouped_persistent(dev, fmt, K):
    """More 256 x 256 tiles than CUs with K of at most 64 blocks: the persistent form, experts
    looked up per tile from one wave's prefix sums, rows past an expert's end dropped by the copy
    and store ranges.  bf16 output equals the RNE of the float32 output (the one-tile launch: the
    same sums in the same order); the first, a middle and the last row of every expert match the
    oracle."""
    counts = [3000, 0, 257, 4100, 1, 2555, 0, 6200, 700]
    E, N = len(counts), 1536
    offsets = workloads.offsets_from_counts(counts)
    T = int(offsets[-1])
    x = workloads.activations(T, K, key=(0, 35, 0, T))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, key=35, fmt=fmt)
    y32 = _run(aq, sa, wq, sw, offsets, dev, torch.float32).cpu().numpy().astype(np.float64)
    y16 = bf16_tensor_to_f64(_run(aq, sa, wq, sw, offsets, dev, torch.bfloat16))
    assert np.array_equal(y16, gemm.bf16_rne(y32))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = np.unique([lo, (lo + hi) // 2, hi - 1])
        check_t1(y32[rows], gemm.gemm_ref(aq[rows], sa[rows], wq[e], sw[e], fmt))


@pytest.mark.parametrize("E", [63, 64])
def test_grouped_expert_count_edge(dev, E):
    """63 experts fill one wave pass of the persistent form's expert table (lane 63 holds the
    final offset); 64 take the one-tile launch's multi-pass lookup.  More tiles than CUs, empty
    and one-row experts included; bf16 equals the RNE of the float32 output and the first and
    last row of every expert match the oracle."""
    rng = np.random.default_rng(E)
    counts = rng.integers(150, 450, E)
    counts[[0, 17, E - 1]] = [0, 1, 0]
    N, K = 1536, 1024
    offsets = workloads.offsets_from_counts(counts)
    T = int(offsets[-1])
    x = workloads.activations(T, K, key=(0, 36, 0, T))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, key=36)
    y32 = _run(aq, sa, wq, sw, offsets, dev, torch.float32).cpu().numpy().astype(np.float64)
    y16 = bf16_tensor_to_f64(_run(aq, sa, wq, sw, offsets, dev, torch.bfloat16))
    assert np.array_equal(y16, gemm.bf16_rne(y32))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows = np.unique([lo, hi - 1])
            check_t1(y32[rows], gemm.gemm_ref(aq[rows], sa[rows], wq[e], sw[e]))


def test_check_offsets(dev):
    """The device check of the grouped GEMM's precondition: 0 for valid offsets (empty experts
    included), else 1 + the first index that breaks it."""
    def chk(vals, total):
        return fgb.check_offsets(torch.tensor(vals, dtype=torch.int32, device=dev), total)
    assert chk([0, 3, 3, 10], 10) == 0
    assert chk([0, 0], 0) == 0
    assert chk([1, 3, 3, 10], 10) == 1          # nonzero start
    assert chk([0, 5, 4, 10], 10) == 3          # offsets[2] < offsets[1]
    assert chk([0, 3, 3, 9], 10) == 4           # ends short of total_M
    many = list(range(0, 700, 10))              # 70 experts: several entries per thread
    assert chk(many, 690) == 0
    many[65] = many[64] - 1
    assert chk(many, 690) == 66


@pytest.mark.parametrize("T,N,K", [(300, 384, 896), (4224, 512, 4096)])
def test_single_expert_equals_dense(dev, T, N, K):
    """E = 1 equals the dense GEMM bit for bit where the dense launch does not slice K (at
    (4224, 512, 4096) the grouped launch uses 256 x 256 tiles and the dense one 256 x 128: the
    per-block partials and their order are the same).  A K-sliced dense launch adds its slices'
    float32 partials afterwards, a different summation order, so these shapes keep it whole."""
    assert fgb.gemm_workspace_bytes(T, N, K) == 0
    x = workloads.activations(T, K, key=(0, 32, 0, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(1, N, K, key=5)
    yg = _run(aq, sa, wq, sw, np.array([0, T]), dev, torch.float32)
    yd = fgb.gemm(torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq[0]).to(dev),
                  torch.from_numpy(sw[0]).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(yg, yd)


def test_zipf_routing_reduced_shape(dev):
    """The MoE routing recipe (Zipf(1.1), top-8 of 32) at 512 tokens with small experts."""
    tok, offsets, counts = workloads.moe_routing(tokens=512, E=32, topk=8, key=(0, 33, 9, 0))
    N, K = 256, 384
    T = int(offsets[-1])
    x = workloads.activations(512, K, key=(0, 33, 0, 0))[tok]
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(32, N, K, key=33)
    yref = gemm.grouped_ref(aq, sa, wq, sw, offsets)
    y16 = _run(aq, sa, wq, sw, offsets, dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)
    assert T == 512 * 8 and counts.min() >= 0
