"""Seeded synthetic inputs shared by the oracle's tests, the GPU parity tests and the benchmark.

This module holds no arithmetic of the quantization method itself: it draws random tensors,
rounds them to bf16 (the source precision of the weights and activations), and describes the
workload shapes. Both the CPU oracle and the HIP path consume exactly the bytes produced here.

Recipes
-------
* Activations ("heavy-tail" outliers): x ~ N(0, 1) in float32; exactly round(0.01*M*K)
  positions, drawn without replacement, are multiplied by 20; the result is rounded to bf16
  with round-to-nearest-even.
* Weights: W ~ N(0, 0.02) in float32, rounded to bf16 (RNE).
* MoE routing: each of T tokens picks `topk` distinct experts out of E with probabilities
  p_e proportional to (e+1)^-1.1 (a Zipf(1.1) skew over expert ranks); rows are then sorted
  by expert, giving contiguous per-expert row ranges and int32 offsets [E+1].

Every generator takes a key tuple; the RNG is numpy's PCG64 seeded with
``np.random.default_rng([seed, cfg_id, tensor_id, shape_id])``.
"""
from __future__ import annotations

import numpy as np

GROUP = 128  # activation group / weight block edge (Transformers "Fine-grained FP8", intro)

# ---------------------------------------------------------------------------------------------
# Workload shapes.  (N, K) pairs are output/input features of a linear layer; y = A @ W^T.
# ---------------------------------------------------------------------------------------------
TINY = dict(name="tiny_64x1024x1024", M=64, N=1024, K=1024)

LLAMA3_8B_LINEARS = [  # Llama-3-8B-shaped projections: QKV, O, gate+up, down
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 28672, 4096),
    ("down", 4096, 14336),
]
LLAMA3_8B_PREFILL_M = 4096

DECODE_SHAPES = LLAMA3_8B_LINEARS + [("ds_qa", 24576, 1536), ("ds_down", 7168, 18432)]
DECODE_MS = [1, 8, 32, 64]

DEEPSEEK_V3_LINEARS = [  # DeepSeek-V3-shaped projections, hidden size 7168
    ("q_b", 24576, 1536),
    ("o", 7168, 16384),
    ("gate_up", 36864, 7168),
    ("down", 7168, 18432),
]
DEEPSEEK_V3_PREFILL_M = 8192

MOE = dict(E=32, tokens=4096, topk=8, zipf=1.1,
           gate_up=(4096, 7168), down=(7168, 2048))


def rng(key) -> np.random.Generator:
    return np.random.default_rng(list(int(k) for k in key))


# ---------------------------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ---------------------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; returns uint16 bit patterns.

    Inputs are finite by construction.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------------------------
def activations(M: int, K: int, key=(0, 0, 0, 0), outlier_frac=0.01, outlier_mult=20.0):
    """bf16 bits [M, K] following the heavy-tail activation recipe."""
    g = rng(key)
    x = g.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        idx = g.choice(M * K, size=n_out, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def weights(N: int, K: int, key=(0, 0, 1, 0), std=0.02):
    """bf16 bits [N, K], W ~ N(0, std)."""
    g = rng(key)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w)


def expert_weights(E: int, N: int, K: int, key=(0, 4, 1, 0), std=0.02):
    """bf16 bits [E, N, K]; expert e uses key + (e,)."""
    out = np.empty((E, N, K), dtype=np.uint16)
    for e in range(E):
        out[e] = weights(N, K, key=tuple(key) + (e,), std=std)
    return out


def moe_routing(tokens=4096, E=32, topk=8, zipf=1.1, key=(0, 4, 9, 0)):
    """Zipf-skewed top-k routing.

    Returns (token_of_row [tokens*topk] int64 sorted by expert, offsets [E+1] int32, counts [E]).
    """
    g = rng(key)
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-zipf)
    p /= p.sum()
    choice = np.empty((tokens, topk), dtype=np.int64)
    for t in range(tokens):
        choice[t] = g.choice(E, size=topk, replace=False, p=p)
    expert_of_row = choice.reshape(-1)
    token_of_row = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.argsort(expert_of_row, kind="stable")
    counts = np.bincount(expert_of_row, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return token_of_row[order], offsets, counts


def offsets_from_counts(counts) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


# ---------------------------------------------------------------------------------------------
# Device-side draws of the same recipes (for full-size runs, where host generation of hundreds of
# millions of values would dominate).  torch's seeded generator on the given device; the values
# are bf16 and any host-side check copies back exactly the bytes the device holds.
# ---------------------------------------------------------------------------------------------
def device_bf16(shape, seed: int, device, outliers: bool = True, std: float = 1.0):
    """bf16 tensor: N(0,1) with round(1% of entries) x20 (outliers=True), or N(0, std)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if outliers:
        n = x.numel()
        idx = torch.randperm(n, generator=gen, device=device)[: int(round(0.01 * n))]
        x.view(-1)[idx] *= 20.0
    else:
        x *= std
    return x.to(torch.bfloat16)
