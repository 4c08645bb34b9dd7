"""Helpers for the GPU GEMM parity tests: upload oracle-side operands, tolerance checks."""
import numpy as np
import torch

from oracle import blockquant, gemm


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def sa_device(s: np.ndarray, dev) -> torch.Tensor:
    """Oracle scales [M, KB] -> the library's K-block-major [KB, ld_sa] with ld_sa % 4 == 0."""
    M, KB = s.shape
    ld = max(4, (M + 3) // 4 * 4)
    out = np.zeros((KB, ld), dtype=np.float32)
    out[:, :M] = s.T
    return torch.from_numpy(out).to(dev)


def upload(aq, sa, wq, sw, dev):
    return (torch.from_numpy(np.ascontiguousarray(aq)).to(dev), sa_device(sa, dev),
            torch.from_numpy(np.ascontiguousarray(wq)).to(dev), torch.from_numpy(np.ascontiguousarray(sw)).to(dev))


def oracle_operands(M, N, K, key=0, fmt="f32", x=None, w=None):
    import workloads
    x = workloads.activations(M, K, key=(key, 20, 0, M)) if x is None else x
    w = workloads.weights(N, K, key=(key, 20, 1, N)) if w is None else w
    aq, sa = blockquant.act_quant(x)
    wq, sw = blockquant.weight_quant(w, fmt)
    return aq, sa, wq, sw


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126) - 7)


def check_t1(y32: np.ndarray, yref: np.ndarray):
    """fp32 mode: max |y32 - y_ref| <= 2e-3 * max |y_ref|."""
    scale = np.max(np.abs(yref))
    err = np.max(np.abs(y32.astype(np.float64) - yref))
    assert err <= 2e-3 * scale, (err, scale)
    return err / scale


def check_t2(y16: np.ndarray, yref: np.ndarray):
    """bf16 mode: per element |y16 - y_ref| <= 2e-3 * max |y_ref| + ulp_bf16(y_ref)."""
    scale = np.max(np.abs(yref))
    err = np.abs(y16.astype(np.float64) - yref)
    bound = 2e-3 * scale + ulp_bf16(yref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])
    return float(np.max(err) / scale)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def ref(aq, sa, wq, sw, fmt="f32"):
    return gemm.gemm_ref(aq, sa, wq, sw, fmt)
