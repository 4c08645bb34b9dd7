"""GPU: the decode-sized entry points captured in a HIP graph and replayed.

Callers that cannot allocate capture these calls (the benchmark's decode rows do too).  One graph
holds a fused-quantization GEMM, a K-sliced no-allocation GEMM (library scratch, second launch),
a decode-shaped grouped MoE GEMM, a batched MoE GEMM and a per-channel scaled GEMM; it is
replayed three times with other eager work and synchronizations in between, and every replay's
outputs must equal the eager results bit for bit.  (No call in the graph records a memset.)"""
import numpy as np
import pytest
import torch

import fine_grained_block_amd as fgb
import workloads

pytestmark = pytest.mark.gpu


def _codes(shape, rng):
    codes = np.arange(256, dtype=np.uint8)
    return rng.choice(codes[(codes & 0x7F) != 0x7F], size=shape)


def test_decode_entries_replay_in_a_graph(dev):
    rng = np.random.default_rng(42)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    # fused quantization, M = 4
    x = workloads.device_bf16((4, 2048), 11, dev)
    w1 = t(_codes((1024, 2048), rng))
    s1 = t((rng.uniform(0.25, 4.0, size=(8, 16)) / 448).astype(np.float32))
    # no-allocation GEMM, K-sliced (6144 x 4096 at M = 40 needs partials)
    a2 = t(_codes((40, 4096), rng))
    sa2 = t((rng.uniform(0.25, 4.0, size=(32, 40)) / 448).astype(np.float32))
    w2 = t(_codes((6144, 4096), rng))
    s2 = t((rng.uniform(0.25, 4.0, size=(48, 32)) / 448).astype(np.float32))
    assert fgb.gemm_workspace_bytes(40, 6144, 4096) > 0
    # grouped (24 rows in all) and batched (16-row slots) MoE
    E, N, K = 8, 256, 1024
    wq = t(_codes((E, N, K), rng))
    swq = t((rng.uniform(0.25, 4.0, size=(E, 2, 8)) / 448).astype(np.float32))
    offs = t(workloads.offsets_from_counts(np.array([3, 0, 5, 1, 0, 8, 7, 0])))
    ag = t(_codes((24, K), rng))
    sag = t((rng.uniform(0.25, 4.0, size=(8, 24)) / 448).astype(np.float32))
    ab = t(_codes((E * 16, K), rng))
    sab = t((rng.uniform(0.25, 4.0, size=(8, E * 16)) / 448).astype(np.float32))
    cnt = t(np.array([16, 0, 4, 9, 1, 0, 16, 2], dtype=np.int32))
    # per-channel scaled GEMM, M = 8
    a5 = t(_codes((8, 1024), rng))
    sa5 = t(rng.uniform(0.001, 0.01, size=8).astype(np.float32))
    w5 = t(_codes((512, 1024), rng))
    sw5 = t(rng.uniform(0.001, 0.01, size=512).astype(np.float32))

    outs = [torch.zeros((4, 1024), dtype=torch.float32, device=dev),
            torch.zeros((40, 6144), dtype=torch.float32, device=dev),
            torch.zeros((24, N), dtype=torch.float32, device=dev),
            torch.zeros((E * 16, N), dtype=torch.float32, device=dev),
            torch.zeros((8, 512), dtype=torch.float32, device=dev)]

    def run():
        fgb.gemm_fused_quant(x, w1, s1, out=outs[0])
        fgb.gemm_noalloc(a2, sa2, w2, s2, outs[1])
        fgb.grouped_gemm(ag, sag, wq, swq, offs, out=outs[2])
        fgb.batched_gemm(ab, sab, wq, swq, cnt, 16, out=outs[3])
        fgb.scaled_gemm(a5, sa5, w5, sw5, act_scale="token", out=outs[4])

    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        # other eager work between replays, including a call that uses the same scratch
        fgb.gemm_noalloc(a2[:20], sa2[:, :20], w2, s2, torch.empty((20, 6144), device=dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            if i == 3:  # batched: only the rows of each slot below its count are written
                valid = torch.cat([torch.arange(16, device=dev) < c for c in cnt.tolist()])
                assert torch.equal(o[valid].view(torch.int32), e[valid].view(torch.int32)), (rep, i)
            else:
                assert torch.equal(o.view(torch.int32), e.view(torch.int32)), (rep, i)
