"""GPU parity for the rows just above the decode sizes, against the oracle, through the C-ABI:
65-128 rows on the shared-ring decode kernel with 128 activation rows (K <= 8192), and the K-sliced
prefill launch (longer rows, or M > 128, with too few output tiles to occupy the CUs).

Each slice multiplies its K-blocks into a float32 partial tile; a second launch adds the slices in
order.  The oracle's result is the same sum over K-blocks (Transformers "Fine-grained FP8", intro:
the 1x128 activation groups and 128x128 weight blocks), so the tolerances are those of every
GEMM test: float32 max|y - y_ref| <= 2e-3 max|y_ref|, bf16 per element 2e-3 max|y_ref| + 1 ulp.
"""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, oracle_operands, ref, upload
from tests.test_gpu_fullsize import _bits, _idx, _pick

pytestmark = pytest.mark.gpu


# (M, N, K): 256x128 tiles with 4 slices; 33 K-blocks in 7 slices of 5 (the last one 3);
# 3 slices of 4 blocks; 128x128 tiles (N % 256 != 0); 3 tile-rows with a ragged last one
SHAPES = [(130, 512, 2048), (160, 768, 4224), (256, 1024, 1536), (200, 1152, 1024), (300, 2048, 2048)]

# (M, N, K) on the 128-row decode kernel: 2 K slices; 4 slices; 6 slices; 4 slices of 32 weight
# blocks; one K-block, unsliced; 37 K-blocks in slices of 10 (the last one 7)
DECODE_128 = [(65, 1024, 2048), (96, 2048, 4096), (128, 512, 6144), (100, 4096, 4096), (128, 256, 128),
              (77, 1280, 4736)]


@pytest.mark.parametrize("M,N,K", DECODE_128)
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_128_rows_parity(dev, M, N, K, fmt):
    ops = oracle_operands(M, N, K, key=6, fmt=fmt)
    yref = ref(*ops, fmt=fmt)
    aq, sa, wq, sw = upload(*ops, dev)
    y32 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    y16 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y32 = y32.cpu().numpy()
    check_t1(y32, yref)
    check_t2(bf16_tensor_to_f64(y16), yref)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_sliced_parity(dev, M, N, K, fmt):
    assert fgb.gemm_workspace_bytes(M, N, K) > 0, "shape expected to take the K-sliced launch"
    ops = oracle_operands(M, N, K, key=7, fmt=fmt)
    yref = ref(*ops, fmt=fmt)
    aq, sa, wq, sw = upload(*ops, dev)
    y32 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    y16 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y32 = y32.cpu().numpy()
    check_t1(y32, yref)
    check_t2(bf16_tensor_to_f64(y16), yref)
    # the bf16 output is the RNE of the same float32 sums (same plan, same slice order)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))


def test_sliced_exact_integers(dev):
    """All scales 1 and every partial and total sum an integer below 2^24: float32 output equal
    to the oracle bit for bit, whatever the slicing."""
    M, N, K = 192, 1024, 4096
    assert fgb.gemm_workspace_bytes(M, N, K) > 0
    rng = np.random.default_rng(11)
    ints = np.array([-3, -2, -1, 0, 1, 2, 3], dtype=np.float32)
    A = rng.choice(ints, size=(M, K))
    W = rng.choice(ints, size=(N, K))
    A[:, ::128] = 448.0
    W[:, 32::128] = 448.0
    aq, sa = blockquant.act_quant(A)
    wq, sw = blockquant.weight_quant(W)
    assert np.all(sa == 1) and np.all(sw == 1)
    yref = gemm.gemm_ref(aq, sa, wq, sw)
    assert np.all(np.abs(yref) < 2 ** 24)
    d = upload(aq, sa, wq, sw, dev)
    y32 = fgb.gemm(*d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y32.cpu().numpy().astype(np.float64), yref)


def test_sliced_strides_guards_and_repeats(dev):
    """Row pitches above the row lengths (a_q, s_a, y), guard bytes around the output, a
    workspace that starts with garbage, and repeated calls: bit-equal to the dense layout, the
    guards intact, every repeat identical."""
    M, N, K = 160, 1280, 3072
    need = fgb.gemm_workspace_bytes(M, N, K)
    assert need > 0
    ops = oracle_operands(M, N, K, key=8)
    aq, sa, wq, sw = upload(*ops, dev)
    dense = fgb.gemm(aq, sa, wq, sw)
    a_pad = torch.zeros((M, K + 256), dtype=torch.uint8, device=dev)
    a_pad[:, :K] = aq
    sa_pad = torch.zeros((K // 128, sa.shape[1] + 64), dtype=torch.float32, device=dev)
    sa_pad[:, :sa.shape[1]] = sa
    guard = torch.full((M + 2, N + 64), -12288.0, dtype=torch.bfloat16, device=dev)
    y = guard[1:M + 1, :N]
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    outs = []
    for _ in range(3):
        fgb.gemm(a_pad[:, :K], sa_pad, wq, sw, out=y, workspace=ws.view(torch.uint8))
        torch.cuda.synchronize()
        outs.append(y.clone())
    for o in outs:
        assert torch.equal(o.view(torch.int16), dense.view(torch.int16))
    g = guard.float()
    assert torch.all(g[0] == -12288.0) and torch.all(g[M + 1] == -12288.0) and torch.all(g[:, N:] == -12288.0)
    check_t2(bf16_tensor_to_f64(dense), ref(*ops))


@pytest.mark.parametrize("name,N,K", workloads.DECODE_SHAPES, ids=[s[0] for s in workloads.DECODE_SHAPES])
def test_rows_above_decode_full_shapes(dev, name, N, K):
    """The full decode weight shapes at M = 65 and 128 (the 128-row decode kernel where K <= 8192,
    else K-sliced prefill tiles) and 256 and 512 (prefill tiles, K-sliced where they leave most
    CUs idle): batched decode and short prefill
    chunks, quantized on the device as in the benchmark.  Sampled rows and weight blocks against
    the oracle, and every output tile in place (a permutation of the weight blocks permutes the
    output columns bit for bit)."""
    seed = sum(map(ord, name)) + 900
    w = workloads.device_bf16((N, K), seed, dev, outliers=False, std=0.02)
    wq, sw = fgb.quantize_weight(w)
    rng = np.random.default_rng(seed)
    _, cols = _pick(rng, 1, N)
    wq_s, sw_s = blockquant.weight_quant(_bits(w[_idx(cols, dev)]), "f32")
    del w
    pb = _idx(rng.permutation(N // 128), dev)
    wq_p = wq.view(N // 128, 128, K)[pb].reshape(N, K).contiguous()
    sw_p = sw[pb].contiguous()
    for M in (65, 128, 256, 512):
        print(f"{name} M={M} workspace={fgb.gemm_workspace_bytes(M, N, K)}", flush=True)
        x = workloads.device_bf16((M, K), seed + M, dev)
        q, sa = fgb.quantize(x)
        y = fgb.gemm(q, sa, wq, sw)
        y_w = fgb.gemm(q, sa, wq_p, sw_p)
        torch.cuda.synchronize()
        assert torch.equal(y_w.view(torch.int16), y.view(M, N // 128, 128)[:, pb].reshape(M, N).view(torch.int16)), M
        rows, _ = _pick(rng, M, N, nrows=32)
        aq, sa_o = blockquant.act_quant(_bits(x[_idx(rows, dev)]))
        yref = gemm.gemm_ref(aq, sa_o, wq_s, sw_s, "f32")
        check_t2(bf16_tensor_to_f64(y[_idx(rows, dev)][:, _idx(cols, dev)]), yref)


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(65, 701)), 128 * int(rng.integers(1, 17)), 128 * int(rng.integers(1, 41)),
             "f32" if i % 2 == 0 else "ue8m0") for i in range(n)]


@pytest.mark.parametrize("M,N,K,fmt", _random_shapes(24, 2024))
def test_random_shapes_around_the_routes(dev, M, N, K, fmt):
    """Seeded random shapes across the 128-row decode route, the K-sliced prefill launch and the
    unsliced tiles (M 65-700, N up to 2048, K up to 5120, either scale format) against the
    oracle, float32 and bf16."""
    ops = oracle_operands(M, N, K, key=M + N + K, fmt=fmt)
    yref = ref(*ops, fmt=fmt)
    d = upload(*ops, dev)
    y32 = fgb.gemm(*d, out_dtype=torch.float32)
    y16 = fgb.gemm(*d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y32 = y32.cpu().numpy()
    check_t1(y32, yref)
    check_t2(bf16_tensor_to_f64(y16), yref)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))
