"""Benchmark: fine-grained FP8 W8A8 linears on one MI355X.

A step is one pass of the hot path over the DeepSeek-V3-shaped prefill batch (M = 8192 tokens,
the largest single-GPU configuration): for each of the four projections (q_b 24576x1536,
o 7168x16384, gate+up 36864x7168, down 7168x18432) the bf16 activations are quantized
dynamically (1x128 groups, float32 scales) and the block-scaled FP8 GEMM with UE8M0 (power-of-two)
128x128 weight scales produces bf16 outputs.  Weights are quantized once beforehand (offline,
untimed); activations are resident in HBM when the timed region starts.

Prints ONE JSON line.  `value` is the whole step's useful GEMM throughput (2*M*N*K summed over
the four projections, divided by the step time, quantization included).  `roofline` is for the
dominant kernel (the prefill GEMM), from HIP events recorded around every GEMM call on the
launch stream inside the timed region.  `cpu_baseline` times the CPU oracle on a bounded sample
of the same workload.  `extra` carries the other rows of the hot path (the Llama-3-8B prefill
step, decode, grouped MoE, quantization bandwidth), each timed on its own.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
MALL_BYTES = 256 << 20
SMALL_PREFILL_MS = (65, 128, 256, 512)  # rows just above the decode sizes


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--suite", choices=["step", "all"], default="all",
                   help="'step': only the headline step; 'all': also the Llama-3-8B step, decode, cold UE8M0 "
                        "prefill calls, MoE, quant")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2048, help="tokens in the oracle sample")
    p.add_argument("--cpu-cols", type=int, default=2048, help="output features per projection in the oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 1 GiB device copy first (reference for HBM byte counters)")
    p.add_argument("--derive-traffic", metavar="PMC_DIR",
                   help="CPU only: read PMC_DIR/{FETCH_SIZE,WRITE_SIZE}/run_counter_collection.csv from "
                        "rocprofv3 --pmc runs of '--suite step --copy-calibration' and write "
                        "profiles/traffic.json")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fine_grained_block_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def derive_traffic(pmc_dir: str, names=None) -> dict:
    """HBM bytes per prefill-GEMM call of the headline step from two rocprofv3 counter runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by 1 GiB over what the same
    counter read for the 1 GiB device copy (__amd_rocclr_copyBuffer) of the same run.  A
    projection's GEMM call is every GEMM dispatch between its act_quant dispatch and the next one
    (a call can be two dispatches: 256x256 and 256x128 tiles); the projections repeat in step
    order.
    """
    import collections
    import csv

    if names is None:
        import workloads
        names = tuple(n for n, _, _ in workloads.DEEPSEEK_V3_LINEARS)
    P = len(names)

    def load(counter):
        per = collections.OrderedDict()
        with open(os.path.join(pmc_dir, counter, "run_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
        return per

    out = {"kernel_source_hash": kernel_source_hash(), "per_projection": {}}
    per_call = 0.0
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = load(counter)
        copy_kib = [v for k, v in d.items() if "copyBuffer" in k[1]]
        if len(copy_kib) != 1:
            raise SystemExit(f"{counter}: expected one 1 GiB copy dispatch, found {len(copy_kib)}")
        factor = (1 << 20) / copy_kib[0]
        out[counter.lower() + "_copy_factor"] = round(factor, 5)
        calls, disp = [], []
        for (did, name), v in sorted(d.items()):
            if "act_quant" in name:
                calls.append(0.0)
                disp.append(0)
            elif "gemm_prefill" in name and calls:
                calls[-1] += v * 1024 * factor
                disp[-1] += 1
        if not calls or len(calls) % P:
            raise SystemExit(f"{counter}: {len(calls)} projection calls, expected whole steps of {P}")
        for i, nm in enumerate(names):
            vals = calls[i::P]
            e = out["per_projection"].setdefault(nm, {})
            e[counter.lower() + "_bytes"] = round(sum(vals) / len(vals))
            e["dispatches"] = disp[i]
        per_call += sum(calls) / len(calls)
    out["gemm_prefill_hbm_bytes_per_call"] = round(per_call)
    out["note"] = ("calibrated HBM fetch + write bytes per prefill-GEMM call of the headline step, mean "
                   "over its projections' calls")
    return out


def _dev_inputs(torch, fgb, workloads, linears, M, scale_fmt, seed0, dev, host_rows=0, host_cols=0):
    """Per projection: bf16 activations [M, K] and quantized weights (offline), drawn on the device
    with seeded generators; optionally the first host_rows activation rows and host_cols weight rows
    copied back as bf16 bit patterns (for the CPU baseline's sample)."""
    import numpy as np
    layers, host = [], []
    for i, (name, N, K) in enumerate(linears):
        w = workloads.device_bf16((N, K), seed0 + 2 * i + 1, dev, outliers=False, std=0.02)
        wq, sw = fgb.quantize_weight(w, scale_fmt)  # offline
        x = workloads.device_bf16((M, K), seed0 + 2 * i, dev)
        if host_rows:
            host.append((x[:host_rows].view(torch.int16).cpu().numpy().view(np.uint16),
                         w[:host_cols].view(torch.int16).cpu().numpy().view(np.uint16)))
        del w
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        layers.append(dict(name=name, N=N, K=K, x=x, wq=wq, sw=sw, q=q, sa=sa, y=y))
    torch.cuda.synchronize()
    return layers, host


def run_step(torch, fgb, layers, M, steps, warmup):
    """Time `steps` back-to-back steps (act_quant + GEMM per projection) after `warmup` untimed
    ones; HIP events around every call on the launch stream give the per-call times."""
    def step(ev=None):
        for j, L in enumerate(layers):
            if ev is not None:
                ev[j][0].record()
            fgb.quantize(L["x"], out=(L["q"], L["sa"]))
            if ev is not None:
                ev[j][1].record()
            fgb.gemm(L["q"], L["sa"], L["wq"], L["sw"], out=L["y"])
            if ev is not None:
                ev[j][2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers] for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        step(evs[s])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    gemm_ms = [sum(evs[s][j][1].elapsed_time(evs[s][j][2]) for s in range(steps)) / steps for j in range(len(layers))]
    quant_ms = [sum(evs[s][j][0].elapsed_time(evs[s][j][1]) for s in range(steps)) / steps for j in range(len(layers))]
    flops = [2.0 * M * L["N"] * L["K"] for L in layers]
    qbytes = [3.03125 * M * L["K"] for L in layers]
    per = {}
    for L, g, q, f, b in zip(layers, gemm_ms, quant_ms, flops, qbytes):
        per[L["name"]] = dict(N=L["N"], K=L["K"], gemm_us=round(g * 1e3, 1), gemm_tflops=round(f / g / 1e9, 1),
                              frac_mfma=round(f / g / 1e9 / PEAK_FP8_TFLOPS, 3),
                              quant_us=round(q * 1e3, 1), quant_gbs=round(b / q / 1e6, 1))
    return dict(M=M, ms_step=ms_step, wall_s=wall, gemm_ms=gemm_ms, quant_ms=quant_ms, flops=flops,
                qbytes=qbytes, per=per)


def headline_step(args, torch, fgb, workloads):
    """The DeepSeek-V3-shaped step (M = 8192, UE8M0 weight scales)."""
    dev = torch.device("cuda:0")
    M = workloads.DEEPSEEK_V3_PREFILL_M
    want_host = not args.no_cpu_baseline
    layers, host = _dev_inputs(torch, fgb, workloads, workloads.DEEPSEEK_V3_LINEARS, M, "ue8m0", 4000, dev,
                               args.cpu_rows if want_host else 0, args.cpu_cols if want_host else 0)
    res = run_step(torch, fgb, layers, M, args.steps, args.warmup)
    del layers
    torch.cuda.empty_cache()
    res["host_sample"] = host
    return res


def llama_step(args, torch, fgb, workloads):
    """The Llama-3-8B-shaped step (M = 4096, float32 weight scales), reported in `extra`."""
    dev = torch.device("cuda:0")
    M = workloads.LLAMA3_8B_PREFILL_M
    layers, _ = _dev_inputs(torch, fgb, workloads, workloads.LLAMA3_8B_LINEARS, M, "float", 3000, dev)
    res = run_step(torch, fgb, layers, M, args.steps, args.warmup)
    del layers
    torch.cuda.empty_cache()
    return dict(ms_per_step=round(res["ms_step"], 4),
                tflops=round(sum(res["flops"]) / (res["ms_step"] * 1e-3) / 1e12, 1),
                gemm_frac_mfma=round(sum(res["flops"]) / (sum(res["gemm_ms"]) * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                per_projection=res["per"])


# ---------------------------------------------------------------------------------------------
def _graph_time(torch, fn, reps):
    """Capture `reps` calls of fn(i) in a HIP graph, replay it, return microseconds per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(2):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (3 * reps)


def _event_time(torch, fn, reps, flush=None):
    ts = []
    for i in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def extra_suites(torch, fgb, workloads, np):
    dev = torch.device("cuda:0")
    seeds = iter(range(1000, 1000000))

    def next_seed():
        return next(seeds)

    out = {}
    # read-only cache flush: a sum over 512 MB of other data (twice the 256 MB MALL) evicts the
    # operands without leaving dirty lines that would drain during the next timed call
    flush_buf = torch.zeros(128 << 20, dtype=torch.float32, device=dev)

    def flush():
        flush_buf.sum()

    # decode — hipGraph loop over rotating weight copies (> 2x MALL in total)
    dec, fused, fp8dyn, small = {}, {}, {}, {}
    for (name, N, K) in workloads.DECODE_SHAPES:
        w = workloads.device_bf16((N, K), next_seed(), dev, outliers=False, std=0.02)
        wq0, sw = fgb.quantize_weight(w)
        wc0, swc = fgb.quantize_weight_per_channel(w)  # FP8_DYNAMIC weights (per channel)
        del w
        copies = max(2, -(-2 * MALL_BYTES // (N * K)) + 1)
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        wcs = [wc0] + [wc0.clone() for _ in range(copies - 1)]
        for M in workloads.DECODE_MS:
            x = workloads.device_bf16((M, K), next_seed(), dev)
            q, sa = fgb.quantize(x)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.zeros(max(256, fgb.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
            us = _graph_time(torch, lambda i: fgb.gemm(q, sa, wqs[i % copies], sw, out=y, workspace=ws), 4 * copies)
            byts = N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * K / 128 + 2 * M * N
            dec[f"{name}_{N}x{K}_M{M}"] = dict(us=round(us, 2), gbs=round(byts / us / 1e3, 1),
                                                frac_hbm=round(byts / us / 1e3 / PEAK_HBM_GBS, 3))
            # the same linear from bf16 activations: act_quant + GEMM (two launches) against the
            # GEMM that quantizes the activations itself (one launch)
            two = _graph_time(torch, lambda i: (fgb.quantize(x, out=(q, sa)),
                                                fgb.gemm(q, sa, wqs[i % copies], sw, out=y, workspace=ws)), 4 * copies)
            fws = torch.zeros(max(256, fgb.gemm_fused_quant_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
            one = _graph_time(torch, lambda i: fgb.gemm_fused_quant(x, wqs[i % copies], sw, out=y, workspace=fws),
                              4 * copies)
            fbytes = N * K + 4 * (N // 128) * (K // 128) + 2 * M * K + 2 * M * N
            fused[f"{name}_{N}x{K}_M{M}"] = dict(quant_plus_gemm_us=round(two, 2), fused_us=round(one, 2),
                                                 fused_frac_hbm=round(fbytes / one / 1e3 / PEAK_HBM_GBS, 3))
            # FP8_DYNAMIC: per-token activation and per-channel weight scales, E4M3
            qt, st = fgb.quantize_per_token(x)
            tdyn = _graph_time(torch, lambda i: fgb.scaled_gemm(qt, st, wcs[i % copies], swc, act_scale="token",
                                                                out=y, workspace=ws), 4 * copies)
            dbytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
            fp8dyn[f"{name}_{N}x{K}_M{M}"] = dict(us=round(tdyn, 2), frac_hbm=round(dbytes / tdyn / 1e3 / PEAK_HBM_GBS, 3))
        # a few rows above the decode sizes (batched decode, short prefill chunks): the prefill
        # kernels, K-sliced where their tiles would leave most CUs idle
        for M in SMALL_PREFILL_MS:
            x = workloads.device_bf16((M, K), next_seed(), dev)
            q, sa = fgb.quantize(x)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.zeros(max(256, fgb.gemm_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dev)
            us = _graph_time(torch, lambda i: fgb.gemm(q, sa, wqs[i % copies], sw, out=y, workspace=ws), 4 * copies)
            byts = N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * K / 128 + 2 * M * N
            small[f"{name}_{N}x{K}_M{M}"] = dict(us=round(us, 2), k_slices=fgb.gemm_workspace_bytes(M, N, K) // (4 * M * N) or 1,
                                                  frac_hbm=round(byts / us / 1e3 / PEAK_HBM_GBS, 3),
                                                  frac_mfma=round(2 * M * N * K / us / 1e6 / PEAK_FP8_TFLOPS, 3))
        del wqs, wq0, wcs, wc0
    out["decode"] = dec
    out["decode_fused_quant"] = fused
    out["decode_fp8_dynamic"] = fp8dyn
    out["prefill_small_m"] = small

    # the other schemes at the Llama-3-8B prefill shapes (M = 4096), back to back: FP8_DYNAMIC
    # (per-token activations, per-channel weights, E4M3) and static per-tensor activations with
    # 128x128 weight blocks in E5M2; quantization and GEMM timed per call with HIP events
    for scheme in ("fp8_dynamic_e4m3", "static_tensor_e5m2"):
        M = workloads.LLAMA3_8B_PREFILL_M
        calls = []
        for (name, N, K) in workloads.LLAMA3_8B_LINEARS:
            w = workloads.device_bf16((N, K), next_seed(), dev, outliers=False, std=0.02)
            x = workloads.device_bf16((M, K), next_seed(), dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            if scheme == "fp8_dynamic_e4m3":
                wq, sw = fgb.quantize_weight_per_channel(w)
                q = torch.empty((M, K), dtype=torch.uint8, device=dev)
                sa = torch.empty((M,), dtype=torch.float32, device=dev)
                quant = (lambda x=x, q=q, sa=sa: fgb.quantize_per_token(x, out=(q, sa)))
                mm = (lambda q=q, sa=sa, wq=wq, sw=sw, y=y: fgb.scaled_gemm(q, sa, wq, sw, act_scale="token", out=y))
            else:
                wq, sw = fgb.quantize_weight(w, "float", code="e5m2")
                q = torch.empty((M, K), dtype=torch.uint8, device=dev)
                sa = torch.tensor([float(x.float().abs().max()) / 57344.0], dtype=torch.float32, device=dev)
                quant = (lambda x=x, q=q, sa=sa: fgb.quantize_static(x, sa, "e5m2", out=q))
                mm = (lambda q=q, sa=sa, wq=wq, sw=sw, y=y: fgb.scaled_gemm(q, sa, wq, sw, act_scale="tensor",
                                                                           code="e5m2", out=y))
            del w
            calls.append((name, N, K, quant, mm, (x, q, sa, wq, sw, y)))
        res = {}
        ev = {n: ([], []) for n, *_ in calls}
        for rep in range(8):
            for (name, N, K, quant, mm, _) in calls:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record(); quant(); e[1].record(); mm(); e[2].record()
                if rep >= 3:
                    ev[name][0].append(e)
        torch.cuda.synchronize()
        for (name, N, K, *_r) in calls:
            qs = sorted(e[0].elapsed_time(e[1]) for e in ev[name][0])
            gs = sorted(e[1].elapsed_time(e[2]) for e in ev[name][0])
            g_us, q_us = gs[len(gs) // 2] * 1e3, qs[len(qs) // 2] * 1e3
            f = 2.0 * M * N * K
            res[f"{name}_{N}x{K}"] = dict(gemm_us=round(g_us, 1), tflops=round(f / g_us / 1e6, 1),
                                          frac_mfma=round(f / g_us / 1e6 / PEAK_FP8_TFLOPS, 3), quant_us=round(q_us, 1),
                                          quant_gbs=round(3.0 * M * K / q_us / 1e3, 1))
        out[f"{scheme}_m4096"] = res
        del calls

    # DeepSeek-V3-shaped prefill with UE8M0 weight scales (M = 8192), each call alone with cold
    # caches (the headline step runs the same calls back to back)
    ds = {}
    M = workloads.DEEPSEEK_V3_PREFILL_M
    for (name, N, K) in workloads.DEEPSEEK_V3_LINEARS:
        w = workloads.device_bf16((N, K), next_seed(), dev, outliers=False, std=0.02)
        wq, sw = fgb.quantize_weight(w, "ue8m0")
        del w
        x = workloads.device_bf16((M, K), next_seed(), dev)
        q, sa = fgb.quantize(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = _event_time(torch, lambda i: fgb.gemm(q, sa, wq, sw, out=y), 5, flush)
        f = 2.0 * M * N * K
        ds[f"{name}_{N}x{K}"] = dict(us=round(us, 1), tflops=round(f / us / 1e6, 1), frac_mfma=round(f / us / 1e6 / PEAK_FP8_TFLOPS, 3))
        del wq, x, q, y
    out["prefill_ue8m0_m8192_cold"] = ds

    # MoE grouped GEMM: 32 experts, 4096 tokens top-8 Zipf(1.1)
    moe = {}
    tok, offsets, counts = workloads.moe_routing()
    off_d = torch.from_numpy(offsets).to(dev)
    T = int(offsets[-1])
    for nm, (N, K) in [("gate_up", workloads.MOE["gate_up"]), ("down", workloads.MOE["down"])]:
        w = workloads.device_bf16((32 * N, K), next_seed(), dev, outliers=False, std=0.02)
        wq, sw = fgb.quantize_weight(w)  # 128-row blocks never straddle experts (N % 128 == 0)
        del w
        wq = wq.view(32, N, K)
        sw = sw.view(32, N // 128, K // 128)
        x = workloads.device_bf16((T, K), next_seed(), dev)
        q, sa = fgb.quantize(x)
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        us = _event_time(torch, lambda i: fgb.grouped_gemm(q, sa, wq, sw, off_d, out=y), 5, flush)
        f = 2.0 * T * N * K
        moe[f"{nm}_{N}x{K}"] = dict(us=round(us, 1), tflops=round(f / us / 1e6, 1), frac_mfma=round(f / us / 1e6 / PEAK_FP8_TFLOPS, 3))
        del wq, x, q, y
    moe["expert_rows_max_min"] = [int(counts.max()), int(counts.min())]
    out["moe_grouped_e32"] = moe

    # decode-shaped MoE (32 experts, top-8 Zipf routing of a few tokens): the grouped layout with
    # 8 or 64 rows in all, and the masked batched layout with 64-row slots for 64 tokens; hipGraph
    # loop alternating two copies of the expert weights (> 2x the MALL); bytes = the routed
    # experts' weights and scales + activations, scales and outputs of the routed rows
    mdec = {}
    for nm, (N, K) in [("gate_up", workloads.MOE["gate_up"]), ("down", workloads.MOE["down"])]:
        w = workloads.device_bf16((32 * N, K), next_seed(), dev, outliers=False, std=0.02)
        wq, sw = fgb.quantize_weight(w)
        del w
        wqs = [wq.view(32, N, K), wq.clone().view(32, N, K)]
        sw = sw.view(32, N // 128, K // 128)
        for tokens in (1, 8, 64):
            _, offs, cnts = workloads.moe_routing(tokens=tokens, key=(0, 9, tokens, 1))
            routed = int((cnts > 0).sum())
            T = int(offs[-1])
            if tokens <= 8:
                x = workloads.device_bf16((T, K), next_seed(), dev)
                q, sa = fgb.quantize(x)
                y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
                off_t = torch.from_numpy(offs).to(dev)
                us = _graph_time(torch, lambda i: fgb.grouped_gemm(q, sa, wqs[i % 2], sw, off_t, out=y), 8)
                key = f"grouped_{nm}_{N}x{K}_T{tokens}_rows{T}"
            else:
                slot = 64
                x = workloads.device_bf16((32 * slot, K), next_seed(), dev)
                q, sa = fgb.quantize(x)
                y = torch.empty((32 * slot, N), dtype=torch.bfloat16, device=dev)
                cnt_t = torch.from_numpy(np.minimum(cnts, slot).astype(np.int32)).to(dev)
                T = int(np.minimum(cnts, slot).sum())
                us = _graph_time(torch, lambda i: fgb.batched_gemm(q, sa, wqs[i % 2], sw, cnt_t, slot, out=y), 8)
                key = f"batched_{nm}_{N}x{K}_T{tokens}_slot{slot}_rows{T}"
            byts = routed * (N * K + 4 * (N // 128) * (K // 128)) + T * (K + 4 * K / 128 + 2 * N)
            mdec[key] = dict(us=round(us, 2), routed_experts=routed, gbs=round(byts / us / 1e3, 1),
                             frac_hbm=round(byts / us / 1e3 / PEAK_HBM_GBS, 3))
        del wqs, wq
    out["moe_decode_e32"] = mdec

    # activation quantization bandwidth at the prefill shapes: hipGraph loop over rotating
    # input/output copies whose total exceeds 2x the MALL, so every call streams from HBM
    qb = {}
    for (M, K) in [(4096, 4096), (4096, 14336), (8192, 7168), (8192, 18432), (32768, 7168)]:
        per_call = 3.03125 * M * K
        copies = max(2, int(-(-2 * MALL_BYTES // per_call)) + 1)
        xs = [workloads.device_bf16((M, K), next_seed(), dev) for _ in range(min(copies, 2))]
        xs += [xs[i % 2].clone() for i in range(copies - len(xs))]
        qs = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(copies)]
        sas = [torch.empty((K // 128, M), dtype=torch.float32, device=dev) for _ in range(copies)]
        us = _graph_time(torch, lambda i: fgb.quantize(xs[i % copies], out=(qs[i % copies], sas[i % copies])), 2 * copies)
        qb[f"{M}x{K}"] = dict(us=round(us, 2), gbs=round(per_call / us / 1e3, 1), frac_hbm=round(per_call / us / 1e3 / PEAK_HBM_GBS, 3))
        del xs, qs, sas
    out["act_quant"] = qb
    return out


# ---------------------------------------------------------------------------------------------
def cpu_baseline(args, host_sample, workloads, np):
    """The CPU oracle (as it is) on a bounded sample of the headline step: the first `cpu_rows`
    tokens and the first `cpu_cols` output features of each projection, full K; act_quant +
    gemm_ref with UE8M0 weight scales.  The sample's bf16 bytes are those the GPU step used.
    Weight quantization of the sampled rows is offline (untimed), as on the GPU."""
    from oracle import blockquant, gemm
    R, C = args.cpu_rows, args.cpu_cols
    prepared = []
    for (x, w), (name, N, K) in zip(host_sample, workloads.DEEPSEEK_V3_LINEARS):
        wq, sw = blockquant.weight_quant(w, "ue8m0")
        prepared.append((x, wq, sw, K))
    t0 = time.perf_counter()
    flops = 0.0
    for x, wq, sw, K in prepared:
        aq, sa = blockquant.act_quant(x)
        gemm.gemm_ref(aq, sa, wq, sw, "ue8m0")
        flops += 2.0 * R * C * K
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=min(cores, threads), kind="oracle",
                sample=f"first {R} tokens x first {C} output features of each of the 4 DeepSeek-V3-shaped "
                       f"projections at M = 8192, full K, UE8M0 weight scales (act_quant + exact-partial "
                       f"float64 gemm_ref); {flops / 1e9:.2f} GFLOP in {dt:.1f} s")


def main():
    args = parse()
    if args.derive_traffic:
        t = derive_traffic(args.derive_traffic)
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
            json.dump(t, fh, indent=1)
            fh.write("\n")
        print(json.dumps(t))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fine_grained_block_amd as fgb
    import workloads

    fgb.lib()
    torch.cuda.init()
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = headline_step(args, torch, fgb, workloads)
    total_flops = sum(res["flops"])
    gemm_total_ms = sum(res["gemm_ms"])
    achieved = total_flops / (gemm_total_ms * 1e-3) / 1e12  # TFLOP/s over the GEMM launches
    extra = {"headline_per_projection": res["per"], "kernel_source_hash": kernel_source_hash()}
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            t = json.load(fh)
        if t.get("kernel_source_hash") == extra["kernel_source_hash"]:
            traffic = t.get("gemm_prefill_hbm_bytes_per_call")
    if args.suite == "all":
        extra["llama3_8b_prefill_m4096_step"] = llama_step(args, torch, fgb, workloads)
        extra.update(extra_suites(torch, fgb, workloads, np))
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, res["host_sample"], workloads, np)
    line = {
        "metric": "block-FP8 GEMM TFLOPS (% of FP8 MFMA peak); quant/decode GB/s (% HBM)",
        "value": round(total_flops / (res["ms_step"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded on the device: x ~ N(0,1) with 1% x20 outliers, W ~ N(0,0.02), bf16)",
        "config": {"workload": "deepseek_v3_prefill_m8192_ue8m0: act_quant_group128 + w8a8_block_gemm for "
                               "q_b 24576x1536, o 7168x16384, gate_up 36864x7168, down 7168x18432; "
                               "UE8M0 128x128 weight scales, float32 1x128 activation scales, bf16 out",
                   "M": res["M"], "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
