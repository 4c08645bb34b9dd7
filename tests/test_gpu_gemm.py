"""GPU parity: w8a8_block_gemm (prefill and decode paths) against the oracle.

Operands are quantized by the oracle on the CPU and uploaded, so these tests isolate the GEMM;
the end-to-end tests quantize on the GPU and compare with the oracle run from the same bf16
inputs.  Tolerances: fp32 mode max|y - y_ref| <= 2e-3 max|y_ref|; bf16 mode per element
|y - y_ref| <= 2e-3 max|y_ref| + 1 bf16 ulp of y_ref.
"""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import (bf16_tensor_to_f64, check_t1, check_t2, oracle_operands, ref,
                                to_dev_bf16, upload)

pytestmark = pytest.mark.gpu


def _run(ops, dev, out_dtype):
    aq, sa, wq, sw = upload(*ops, dev)
    y = fgb.gemm(aq, sa, wq, sw, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,N,K", [
    (64, 1024, 1024),                         # tiny config (decode path: M <= 64)
    (65, 256, 256), (128, 128, 128), (200, 384, 640), (300, 1024, 1024), (513, 768, 2048),
    (1, 256, 1024), (8, 512, 384), (32, 1024, 2048), (64, 256, 128), (17, 128, 4096),
])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_gemm_parity(dev, M, N, K, fmt):
    ops = oracle_operands(M, N, K, key=1, fmt=fmt)
    yref = ref(*ops, fmt=fmt)
    y32 = _run(ops, dev, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run(ops, dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)
    # the bf16 epilogue is the RNE of the same float32 accumulators
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))


@pytest.mark.parametrize("M", [1, 33, 64, 130, 512])
def test_exact_integer_case(dev, M):
    """Scales are all exactly 1 and every product sum is an integer below 2^24: the float32
    result must equal the oracle bit for bit, and bf16 must be its RNE."""
    rng = np.random.default_rng(M)
    N, K = 384, 1024
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
    A = rng.choice(ints, size=(M, K))
    W = rng.choice(ints, size=(N, K))
    A[:, ::128] = 448.0
    W[:, 64::128] = -448.0
    aq, sa = blockquant.act_quant(A)
    wq, sw = blockquant.weight_quant(W)
    yref = gemm.gemm_ref(aq, sa, wq, sw)
    assert np.all(sa == 1) and np.all(sw == 1) and np.all(np.abs(yref) < 2 ** 24)
    y32 = _run((aq, sa, wq, sw), dev, torch.float32).cpu().numpy()
    assert np.array_equal(y32.astype(np.float64), yref)
    y16 = _run((aq, sa, wq, sw), dev, torch.bfloat16)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(yref))


def test_homogeneity_in_weight_scales(dev):
    ops = oracle_operands(96, 256, 512, key=2)
    aq, sa, wq, sw = ops
    y1 = _run(ops, dev, torch.float32).cpu().numpy()
    y2 = _run((aq, sa, wq, (sw * np.float32(2)).astype(np.float32)), dev, torch.float32).cpu().numpy()
    assert np.array_equal(y2, 2 * y1)


def test_output_canaries_and_strides(dev):
    """Writes stay inside [M, N] of a wider output buffer (ldy > N); the guard bytes keep
    their pattern."""
    M, N, K = 100, 256, 256
    ops = oracle_operands(M, N, K, key=3)
    aq, sa, wq, sw = upload(*ops, dev)
    for dt in (torch.bfloat16, torch.float32):
        buf = torch.full((M + 2, N + 64), -7.0, dtype=dt, device=dev)
        y = buf[1:M + 1, 8:N + 8]
        fgb.gemm(aq, sa, wq, sw, out=y)
        torch.cuda.synchronize()
        b = buf.float().cpu().numpy()
        assert np.all(b[0] == -7) and np.all(b[M + 1] == -7)
        assert np.all(b[:, :8] == -7) and np.all(b[:, N + 8:] == -7)
        check_t2(b[1:M + 1, 8:N + 8].astype(np.float64), ref(*ops))


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_decode_shapes_reduced(dev, M):
    """Decode path at moderate (N, K), including several K splits."""
    for N, K in [(4096, 4096), (1536, 14336)]:
        ops = oracle_operands(M, N, K, key=4)
        yref = ref(*ops)
        y16 = _run(ops, dev, torch.bfloat16)
        check_t2(bf16_tensor_to_f64(y16), yref)


def test_end_to_end_linear(dev):
    """quantize (GPU) + gemm (GPU) from bf16 inputs against the oracle from the same inputs."""
    M, N, K = 256, 512, 1024
    x = workloads.activations(M, K, key=(0, 5, 0, 0))
    w = workloads.weights(N, K, key=(0, 5, 1, 0))
    wq, sw = fgb.quantize_weight(to_dev_bf16(w, dev))
    y = fgb.linear(to_dev_bf16(x, dev), wq, sw)
    torch.cuda.synchronize()
    yref = ref(*oracle_operands(M, N, K, x=x, w=w))
    check_t2(bf16_tensor_to_f64(y), yref)


def test_empty_m_is_noop(dev):
    aq = torch.empty((0, 256), dtype=torch.uint8, device=dev)
    sa = torch.empty((2, 4), dtype=torch.float32, device=dev)
    wq = torch.zeros((128, 256), dtype=torch.uint8, device=dev)
    sw = torch.ones((1, 2), dtype=torch.float32, device=dev)
    y = fgb.gemm(aq, sa, wq, sw)
    assert y.shape == (0, 128)


def test_rejects_bad_shapes(dev):
    aq = torch.zeros((16, 200), dtype=torch.uint8, device=dev)
    sa = torch.zeros((2, 16), dtype=torch.float32, device=dev)
    wq = torch.zeros((128, 200), dtype=torch.uint8, device=dev)
    sw = torch.ones((1, 2), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="multiple of 128"):
        fgb.gemm(aq, sa, wq, sw)


def test_decode_workspace_reuse_across_shapes(dev):
    """One workspace buffer serves a sequence of K-sliced decode calls of different shapes (its contents
    on entry do not matter)."""
    shapes = [(64, 6144, 4096), (1, 1024, 2048), (33, 4096, 4096), (8, 1536, 14336), (40, 2048, 16384)]
    need = max(fgb.gemm_workspace_bytes(*s) for s in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)  # NaN-patterned on entry
    for rep in range(2):
        for (M, N, K) in shapes:
            ops = oracle_operands(M, N, K, key=6)
            aq, sa, wq, sw = upload(*ops, dev)
            y = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32, workspace=ws)
            torch.cuda.synchronize()
            check_t1(y.cpu().numpy(), ref(*ops))


_RING_W = {}


def _ring_weights(fmt):
    """A 2048 x 24576 weight (exactly 48 MiB of codes with K >= 8192, from which M <= 16 calls take
    the LDS-ring decode kernel): random finite E4M3 codes and random block scales."""
    if fmt not in _RING_W:
        N, K = 2048, 24576
        rng = np.random.default_rng(77)
        codes = np.arange(256, dtype=np.uint8)
        finite = codes[(codes & 0x7F) != 0x7F]
        wq = rng.choice(finite, size=(N, K))
        if fmt == "f32":
            sw = (rng.uniform(0.25, 4.0, size=(N // 128, K // 128)) / 448).astype(np.float32)
        else:
            sw = rng.integers(112, 124, size=(N // 128, K // 128), dtype=np.uint8)
        _RING_W[fmt] = (wq, sw)
    return _RING_W[fmt]


@pytest.mark.parametrize("M", [1, 7, 8, 9, 16])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_large_weight_ring_kernel(dev, M, fmt):
    """M <= 16 with a large weight (the LDS-ring decode kernel), both activation-row stagings
    (M <= 8 and M <= 16); operands are random finite codes and scales."""
    wq, sw = _ring_weights(fmt)
    N, K = wq.shape
    rng = np.random.default_rng(1000 + M)
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    aq = rng.choice(finite, size=(M, K))
    sa = (rng.uniform(0.25, 4.0, size=(M, K // 128)) / 448).astype(np.float32)
    yref = gemm.gemm_ref_fast(aq, sa, wq, sw, fmt)
    y32 = _run((aq, sa, wq, sw), dev, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run((aq, sa, wq, sw), dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)


def _mid_rows_case(dev, M, N, K, fmt):
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    rng = np.random.default_rng(3000 + M + N + K)
    wq = rng.choice(finite, size=(N, K))
    if fmt == "f32":
        sw = (rng.uniform(0.25, 4.0, size=(N // 128, K // 128)) / 448).astype(np.float32)
    else:
        sw = rng.integers(112, 124, size=(N // 128, K // 128), dtype=np.uint8)
    aq = rng.choice(finite, size=(M, K))
    sa = (rng.uniform(0.25, 4.0, size=(M, K // 128)) / 448).astype(np.float32)
    yref = gemm.gemm_ref_fast(aq, sa, wq, sw, fmt)
    y32 = _run((aq, sa, wq, sw), dev, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run((aq, sa, wq, sw), dev, torch.bfloat16)
    check_t2(bf16_tensor_to_f64(y16), yref)


@pytest.mark.parametrize("M", [17, 32, 33, 48, 64])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_mid_rows_ring_kernel(dev, M, fmt):
    """16 < M <= 64 with weights of at most 16 MiB (the per-wave ring kernel with 32 or 64
    activation rows, 4 waves splitting K): 25 K-blocks (ragged split over the waves), 2 blocks
    (N = 16384), 12 blocks; random finite codes and scales, float32 and bf16 outputs."""
    for (N, K) in [(1024, 3200), (16384, 256), (2048, 1536)]:
        _mid_rows_case(dev, M, N, K, fmt)


@pytest.mark.parametrize("M", [17, 32, 33, 48, 64])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_mid_rows_kernel(dev, M, fmt):
    """16 < M <= 64 with weights above 16 MiB (the streaming kernel with an LDS ring shared by a
    workgroup's waves): a K slicing with a ragged last slice shorter than the ring (N = 1024,
    K = 16512: 129 K-blocks in 14 slices of 9 and one of 3), 13 slices of 10 and 8 blocks
    (N = 2048, K = 16384), and a single slice (N = 20480, K = 1024); random finite codes and
    scales, float32 and bf16 outputs."""
    for (N, K) in [(1024, 16512), (2048, 16384), (20480, 1024)]:
        _mid_rows_case(dev, M, N, K, fmt)


@pytest.mark.parametrize("M", [17, 24, 32, 33])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_decode_mid_rows_fewer_waves(dev, M, fmt):
    """At most 32 activation rows with 32-63 K-blocks: workgroups of 2 waves (N = 4096, K = 4608:
    128 workgroups, 36 blocks) or 4 waves (N = 10240, K = 5248: 160 workgroups, 41 blocks, odd
    against the ring depth) over the whole K, one launch; M = 33 takes the 8-wave kernel with K
    slices on the same shapes."""
    for (N, K) in [(4096, 4608), (10240, 5248)]:
        assert (fgb.gemm_workspace_bytes(M, N, K) == 0) == (M <= 32)
        _mid_rows_case(dev, M, N, K, fmt)


@pytest.mark.parametrize("M,N,K", [(1000, 32768, 1024), (1700, 16384, 2048), (4096, 8192, 2048), (520, 65536, 1280)])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_persistent_prefill_tiles(dev, M, N, K, fmt):
    """256 x 256 tiles with more tiles than CUs and K of at most 16 blocks (bf16 output): each
    workgroup walks several tiles, copying the next tile's first block while it stores the
    current one.  Ragged M, tile counts that are and are not multiples of the grid, 8 to 16
    K-blocks, both scale formats (UE8M0 with 10 K-blocks takes the one-tile launch).  Every output
    equals the RNE of the float32-output kernel's (the same sums in the same order), and a sample
    of rows, including every tile's first and last, matches the oracle."""
    ops = oracle_operands(M, N, K, key=9, fmt=fmt)
    aq, sa, wq, sw = upload(*ops, dev)
    y16 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16)
    y32 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y16 = bf16_tensor_to_f64(y16)
    assert np.array_equal(y16, gemm.bf16_rne(y32.cpu().numpy().astype(np.float64)))
    ends = np.arange(0, M, 256)
    rows = np.unique(np.concatenate([ends, np.minimum(ends + 255, M - 1), [M // 2]]))
    aq_o, sa_o, wq_o, sw_o = ops
    check_t2(y16[rows], ref(aq_o[rows], sa_o[rows], wq_o, sw_o, fmt=fmt))


@pytest.mark.parametrize("M", [4096, 4000, 3900])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_split_columns_big_and_half_tiles(dev, M, fmt):
    """N = 6144 at M ~ 4096: the first 4096 output columns run as 256 x 256 tiles and the last
    2048 as 256 x 128 tiles (two launches on offset weight rows, scale rows and output
    columns).  Rows across the tile-rows (and the ragged last one: 160 or 60 rows, where the
    waves of the empty 64-row quarters skip their MFMAs) are checked against the oracle over
    all columns, so both parts and their boundary are covered; bf16 output is the RNE of the
    float32 output."""
    N, K = 6144, 1024
    ops = oracle_operands(M, N, K, key=12, fmt=fmt)
    aq, sa, wq, sw = upload(*ops, dev)
    y32 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    y16 = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y32 = y32.cpu().numpy().astype(np.float64)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32))
    rows = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(127, M, 256), [M - 1]]))
    aq_o, sa_o, wq_o, sw_o = ops
    check_t1(y32[rows], ref(aq_o[rows], sa_o[rows], wq_o, sw_o, fmt=fmt))


@pytest.mark.parametrize("M,N,K", [(1000, 32768, 1024), (3900, 6144, 1024)])
def test_persistent_and_split_paths_respect_strides(dev, M, N, K):
    """The persistent launch (range-checked stores based at each tile) and the split-column
    launches (offset output columns) write exactly the [M, N] window of a wider output buffer
    (ldy > N): the guard rows and columns keep their pattern, and the window equals the result
    written to a dense output."""
    ops = oracle_operands(M, N, K, key=13)
    aq, sa, wq, sw = upload(*ops, dev)
    dense = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16)
    buf = torch.full((M + 2, N + 64), -7.0, dtype=torch.bfloat16, device=dev)
    fgb.gemm(aq, sa, wq, sw, out=buf[1:M + 1, 8:N + 8])
    torch.cuda.synchronize()
    assert torch.equal(buf[1:M + 1, 8:N + 8], dense)
    assert bool((buf[0] == -7).all()) and bool((buf[M + 1] == -7).all())
    assert bool((buf[:, :8] == -7).all()) and bool((buf[:, N + 8:] == -7).all())


def test_repeated_runs_are_bitwise_identical(dev):
    """Every path sums in a fixed order, so repeated runs must agree bit for bit; a race between
    the LDS copies and the reads of a stage (or between workgroups) would show up as run-to-run
    differences.  Each shape runs six times with the caches flushed before every other run:
    256x256 and 256x128 prefill tiles, the persistent 256x256 form (bf16 output, two tiles per
    workgroup), the 128x128 tile (N % 256 != 0), the decode ring kernel
    (M <= 16, 48 MiB of weights with K >= 8192), the M <= 16 register kernel with its per-wave LDS
    reorder (small and large weights), the 16 < M <= 64 kernel with a K slicing and its
    reduction, and the grouped GEMM."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)

    def codes(shape):
        c = torch.randint(0, 256, shape, generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
        return torch.where((c & 0x7F) == 0x7F, c ^ 1, c)  # finite E4M3 codes only

    def scales(shape):
        return torch.rand(shape, generator=gen, device=dev) * (2.0 / 448) + 0.25 / 448

    cases = [(4096, 4096, 2048), (4096, 6144, 4096), (1024, 1152, 1024), (8, 2048, 24576), (48, 1024, 3200),
             (4, 6144, 4096), (16, 28672, 4096)]
    for (M, N, K) in cases:
        aq, sa = codes((M, K)), scales((K // 128, M))
        wq, sw = codes((N, K)), scales((N // 128, K // 128))
        outs = []
        for i in range(6):
            if i % 2:
                flush.fill_(1)
            outs.append(fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32))
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32)), (M, N, K)
    # bf16 output with more 256 x 256 tiles than CUs: the persistent form
    M, N, K = 2048, 16384, 2048
    aq, sa = codes((M, K)), scales((K // 128, M))
    wq, sw = codes((N, K)), scales((N // 128, K // 128))
    outs = []
    for i in range(6):
        if i % 2:
            flush.fill_(1)
        outs.append(fgb.gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), (M, N, K, "bf16")
    E, N, K = 8, 1024, 2048
    counts = [700, 0, 1, 255, 256, 257, 1500, 63]  # 3032 rows: the scale rows stay 16-byte aligned
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
    T = int(sum(counts))
    aq, sa = codes((T, K)), scales((K // 128, T))
    wq, sw = codes((E, N, K)), scales((E, N // 128, K // 128))
    outs = []
    for i in range(6):
        if i % 2:
            flush.fill_(1)
        outs.append(fgb.grouped_gemm(aq, sa, wq, sw, offsets, out_dtype=torch.float32))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32)), "grouped"


def _random_operands(M, N, K, fmt, seed):
    """Random finite E4M3 codes and positive scales (no quantization step: the GEMM alone)."""
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    rng = np.random.default_rng(seed)
    aq = rng.choice(finite, size=(M, K))
    wq = rng.choice(finite, size=(N, K))
    sa = (rng.uniform(0.25, 4.0, size=(M, K // 128)) / 448).astype(np.float32)
    if fmt == "f32":
        sw = (rng.uniform(0.25, 4.0, size=(N // 128, K // 128)) / 448).astype(np.float32)
    else:
        sw = rng.integers(112, 124, size=(N // 128, K // 128), dtype=np.uint8)
    return aq, sa, wq, sw


@pytest.mark.parametrize("M", [1, 8, 16, 24, 64, 300])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_maximum_k(dev, M, fmt):
    """K = 32768, the largest K the library accepts (256 K-blocks), on every M-dependent path at
    N = 1024: the decode register kernel (M <= 16), the shared-ring kernel in 26 K slices with
    the ordered reduction (M = 24, 64), prefill tiles (M = 300, the weight-block scales of a tile
    staged at full length)."""
    ops = _random_operands(M, 1024, 32768, fmt, seed=4000 + M)
    yref = gemm.gemm_ref_fast(*ops, fmt)
    y32 = _run(ops, dev, torch.float32).cpu().numpy()
    check_t1(y32, yref)
    y16 = _run(ops, dev, torch.bfloat16)
    assert np.array_equal(bf16_tensor_to_f64(y16), gemm.bf16_rne(y32.astype(np.float64)))


def test_activation_offsets_near_4gib(dev):
    """M * K just below 2^32 (131071 rows of K = 32768, 4 GiB - 32 KiB of activation codes): the
    copies' 32-bit row offsets run up to the limit the library validates.  Codes and scales are
    drawn on the device; sampled rows (the first, both sides of the 2^31-byte offset, the last
    tile's rows, the last) are checked against the oracle on the bytes the device holds."""
    M, N, K = 131071, 256, 32768
    assert M * K < 2 ** 32 <= (M + 1) * K
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    aq = torch.randint(0, 0x7F, (M, K), dtype=torch.uint8, device=dev, generator=g)
    aq |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev, generator=g) << 7
    ld_sa = (M + 3) // 4 * 4
    sa = torch.rand((K // 128, ld_sa), device=dev, generator=g) * (3.75 / 448) + 0.25 / 448
    _, _, wq_np, sw_np = _random_operands(1, N, K, "f32", seed=4100)
    wq, sw = torch.from_numpy(wq_np).to(dev), torch.from_numpy(sw_np).to(dev)
    y = fgb.gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    half = (2 ** 31) // K
    rows = np.unique(np.array([0, 1, half - 1, half, half + 1, M - 256, M - 200, M - 2, M - 1]))
    ridx = torch.from_numpy(rows).to(dev)
    aq_s = aq[ridx].cpu().numpy()
    sa_s = sa[:, ridx].t().contiguous().cpu().numpy()
    yref = gemm.gemm_ref(aq_s, sa_s, wq_np, sw_np, "f32")
    check_t1(y[ridx].cpu().numpy(), yref)


@pytest.mark.parametrize("M", [1, 8, 16, 24, 40, 64])
@pytest.mark.parametrize("N,K", [(1024, 2048), (6144, 4096), (2048, 24576), (1024, 16512)])
def test_decode_strides_and_canaries(dev, M, N, K):
    """Every decode kernel with row pitches above the row lengths (lda = K + 128, ld_sa 12 above M,
    ldy = N + 64): equal bit for bit to the dense-layout call, and the bytes around the output
    untouched.  The shapes reach the register kernel, the LDS-ring kernel (2048 x 24576), the
    per-wave ring for 32/64 rows (1024 x 2048), the 2-wave and the sliced 8-wave shared-ring
    kernels (6144 x 4096, 1024 x 16512)."""
    aq, sa, wq, sw = _random_operands(M, N, K, "f32", seed=4200 + M + N)
    aqd, sad, wqd, swd = upload(aq, sa, wq, sw, dev)
    dense = fgb.gemm(aqd, sad, wqd, swd, out_dtype=torch.float32)
    abuf = torch.zeros((M, K + 128), dtype=torch.uint8, device=dev)
    abuf[:, :K] = aqd
    ld_sa = (M + 3) // 4 * 4 + 12  # (the library takes 16-byte row pitches)
    sbuf = torch.full((K // 128, ld_sa), 7.0, dtype=torch.float32, device=dev)
    sbuf[:, :M] = sad[:, :M]
    ybuf = torch.full((M + 2, N + 64), -7.0, dtype=torch.float32, device=dev)
    fgb.gemm(abuf[:, :K], sbuf, wqd, swd, out=ybuf[1:M + 1, 32:N + 32])
    torch.cuda.synchronize()
    assert torch.equal(ybuf[1:M + 1, 32:N + 32].view(torch.int32), dense.view(torch.int32))
    b = ybuf.cpu().numpy()
    assert np.all(b[0] == -7) and np.all(b[M + 1] == -7)
    assert np.all(b[:, :32] == -7) and np.all(b[:, N + 32:] == -7)
