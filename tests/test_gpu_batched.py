"""GPU parity for the MoE layouts beyond the contiguous prefill case, through the C-ABI:
the masked batched layout [E, max_M] with per-expert counts (fgb_batched_w8a8_block_gemm: the
per-expert weight-streaming kernel for max_M <= 64, the grouped prefill kernel above), and the
grouped layout with at most 64 rows in all (decode-shaped routing: the per-expert streaming
kernel).  Against oracle.gemm.batched_ref / grouped_ref; padding rows of a slot must stay
untouched.  Tolerances as for the dense GEMM."""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads
from oracle import blockquant, gemm
from tests.gemm_helpers import bf16_tensor_to_f64, check_t1, check_t2, sa_device

pytestmark = pytest.mark.gpu


def _experts(E, N, K, fmt, key):
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    rng = np.random.default_rng(key)
    wq = rng.choice(finite, size=(E, N, K))
    if fmt == "f32":
        sw = (rng.uniform(0.25, 4.0, size=(E, N // 128, K // 128)) / 448).astype(np.float32)
    else:
        sw = rng.integers(112, 124, size=(E, N // 128, K // 128), dtype=np.uint8)
    return wq, sw


@pytest.mark.parametrize("max_m", [1, 5, 16, 40, 64, 100, 300])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_batched_masked_layout(dev, max_m, fmt):
    E, N, K = 8, 256, 1024
    rng = np.random.default_rng(max_m)
    counts = rng.integers(0, max_m + 1, size=E)
    counts[0], counts[3] = 0, max_m                     # an empty and a full slot
    x = workloads.activations(E * max_m, K, key=(3, 70, max_m, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, fmt, 100 + max_m)
    yref, valid = gemm.batched_ref(aq, sa, wq, sw, counts, max_m, fmt)
    args = (torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq).to(dev),
            torch.from_numpy(sw).to(dev), torch.from_numpy(counts.astype(np.int32)).to(dev), max_m)
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((E * max_m, N), -7.0, dtype=dt, device=dev)
        fgb.batched_gemm(*args, out=out)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy().astype(np.float64)
        assert np.all(o[~valid] == -7.0), "padding rows were written"
        if valid.any():
            if dt == torch.float32:
                check_t1(o[valid], yref[valid])
            else:
                check_t2(o[valid], yref[valid])


def test_batched_equals_grouped_on_the_same_rows(dev):
    """The batched layout and the contiguous grouped layout agree on every valid row."""
    E, N, K, max_m = 6, 512, 2048, 48
    counts = np.array([48, 0, 3, 17, 1, 30])
    x = workloads.activations(E * max_m, K, key=(3, 71, 0, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, "f32", 7)
    wqd, swd = torch.from_numpy(wq).to(dev), torch.from_numpy(sw).to(dev)
    yb = fgb.batched_gemm(torch.from_numpy(aq).to(dev), sa_device(sa, dev), wqd, swd,
                          torch.from_numpy(counts.astype(np.int32)).to(dev), max_m, out_dtype=torch.float32)
    rows = np.concatenate([np.arange(e * max_m, e * max_m + counts[e]) for e in range(E)])
    offsets = workloads.offsets_from_counts(counts)
    yg = fgb.grouped_gemm(torch.from_numpy(aq[rows]).to(dev), sa_device(sa[rows], dev), wqd, swd,
                          torch.from_numpy(offsets).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    # (grouped with more than 64 rows runs the prefill kernel: a different summation order)
    check_t1(yb.cpu().numpy()[rows], yg.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("tokens", [1, 3, 8])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_grouped_decode_shaped_routing(dev, tokens, fmt):
    """Top-8 routing of a few tokens over 32 experts (Zipf 1.1): at most 64 rows in all, so the
    grouped GEMM streams each routed expert's weights; unrouted experts read nothing."""
    E, N, K = 32, 256, 2048
    _, offsets, counts = workloads.moe_routing(tokens=tokens, E=E, topk=8, key=(3, 72, tokens, 0))
    T = int(offsets[-1])
    assert T == 8 * tokens <= 64
    x = workloads.activations(T, K, key=(3, 73, tokens, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, fmt, 200 + tokens)
    yref = gemm.grouped_ref(aq, sa, wq, sw, offsets, fmt)
    args = (torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq).to(dev),
            torch.from_numpy(sw).to(dev), torch.from_numpy(offsets).to(dev))
    y32 = fgb.grouped_gemm(*args, out_dtype=torch.float32)
    y16 = fgb.grouped_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_t1(y32.cpu().numpy(), yref)
    check_t2(bf16_tensor_to_f64(y16), yref)


def test_grouped_decode_all_rows_in_one_expert(dev):
    E, N, K, T = 16, 512, 1024, 64
    counts = np.zeros(E, dtype=np.int64)
    counts[5] = T
    offsets = workloads.offsets_from_counts(counts)
    x = workloads.activations(T, K, key=(3, 74, 0, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, "f32", 9)
    yref = gemm.grouped_ref(aq, sa, wq, sw, offsets)
    y = fgb.grouped_gemm(torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq).to(dev),
                         torch.from_numpy(sw).to(dev), torch.from_numpy(offsets).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_t1(y.cpu().numpy(), yref)
    # one expert holding every row equals the dense GEMM on that expert's weights
    yd = fgb.gemm(torch.from_numpy(aq).to(dev), sa_device(sa, dev), torch.from_numpy(wq[5]).to(dev),
                  torch.from_numpy(sw[5]).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, yd)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_moe_decode_two_tile_passes(dev, fmt):
    """Experts with more than 16 rows and K of at least 32 blocks: the per-expert streaming kernel
    takes 32 rows per weight pass (two 16-row tiles share each weight fragment).  Slot counts 0,
    16, 17 (a one-row second tile), 33 (a two-tile pass and a one-row pass) and 64; against the
    oracle, bf16 equal to the RNE of float32, padding untouched, and the grouped layout of the
    same rows (33 in all, the same kernel) equal bit for bit."""
    E, N, K, max_m = 5, 256, 4096, 64
    counts = np.array([64, 0, 17, 33, 16])
    x = workloads.activations(E * max_m, K, key=(3, 74, 0, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, fmt, 11)
    yref, valid = gemm.batched_ref(aq, sa, wq, sw, counts, max_m, fmt)
    wqd, swd = torch.from_numpy(wq).to(dev), torch.from_numpy(sw).to(dev)
    args = (torch.from_numpy(aq).to(dev), sa_device(sa, dev), wqd, swd,
            torch.from_numpy(counts.astype(np.int32)).to(dev), max_m)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((E * max_m, N), -7.0, dtype=dt, device=dev)
        fgb.batched_gemm(*args, out=out)
        torch.cuda.synchronize()
        outs[dt] = out
        o = out.float().cpu().numpy().astype(np.float64)
        assert np.all(o[~valid] == -7.0), "padding rows were written"
        (check_t1 if dt == torch.float32 else check_t2)(o[valid], yref[valid])
    y32 = outs[torch.float32].cpu().numpy().astype(np.float64)
    assert np.array_equal(bf16_tensor_to_f64(outs[torch.bfloat16])[valid], gemm.bf16_rne(y32[valid]))
    # experts 2 and 3 alone in the grouped layout (33 rows in all: the same per-expert kernel)
    sub = np.array([0, 0, 17, 33, 0])
    rows = np.concatenate([np.arange(e * max_m, e * max_m + sub[e]) for e in range(E)])
    yg = fgb.grouped_gemm(torch.from_numpy(aq[rows]).to(dev), sa_device(sa[rows], dev), wqd, swd,
                          torch.from_numpy(workloads.offsets_from_counts(sub)).to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(yg.cpu().numpy().astype(np.float64), y32[rows])


@pytest.mark.parametrize("K", [2048, 4096])
def test_moe_decode_strides_and_canaries(dev, K):
    """The per-expert streaming kernel (grouped, 40 rows in all; batched 48-row slots) with row
    pitches above the row lengths (lda = K + 256, ld_sa 8 above the rows, ldy = N + 32): equal
    bit for bit to the dense-layout calls, the bytes around the output untouched."""
    E, N = 6, 512
    counts = np.array([17, 0, 3, 9, 0, 11])
    T = int(counts.sum())
    x = workloads.activations(T, K, key=(3, 75, K, 0))
    aq, sa = blockquant.act_quant(x)
    wq, sw = _experts(E, N, K, "f32", 12)
    wqd, swd = torch.from_numpy(wq).to(dev), torch.from_numpy(sw).to(dev)
    off = torch.from_numpy(workloads.offsets_from_counts(counts)).to(dev)
    aqd, sad = torch.from_numpy(aq).to(dev), sa_device(sa, dev)
    dense = fgb.grouped_gemm(aqd, sad, wqd, swd, off, out_dtype=torch.float32)
    abuf = torch.zeros((T, K + 256), dtype=torch.uint8, device=dev)
    abuf[:, :K] = aqd
    ld = sad.shape[1] + 8
    sbuf = torch.full((K // 128, ld), 3.0, dtype=torch.float32, device=dev)
    sbuf[:, :T] = sad[:, :T]
    ybuf = torch.full((T + 2, N + 32), -7.0, dtype=torch.float32, device=dev)
    fgb.grouped_gemm(abuf[:, :K], sbuf, wqd, swd, off, out=ybuf[1:T + 1, 16:N + 16])
    torch.cuda.synchronize()
    assert torch.equal(ybuf[1:T + 1, 16:N + 16].view(torch.int32), dense.view(torch.int32))
    b = ybuf.cpu().numpy()
    assert np.all(b[0] == -7) and np.all(b[T + 1] == -7) and np.all(b[:, :16] == -7) and np.all(b[:, N + 16:] == -7)
