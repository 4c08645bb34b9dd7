"""ctypes loader for libfgb.so with the argument types of include/fgb.h."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libfgb.so")

SCALE_F32, SCALE_UE8M0 = 0, 1
ACT_SCALE_GROUP128, ACT_SCALE_TOKEN, ACT_SCALE_TENSOR = 0, 1, 2
W_SCALE_BLOCK128, W_SCALE_CHANNEL = 0, 1
OUT_BF16, OUT_F32 = 0, 1
FP8_E4M3, FP8_E5M2, UE8M0, FP8_E4M3_INT = 0, 1, 2, 3

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_SIGS = {
    "fgb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fgb_abi_version": (ctypes.c_int, []),
    "fgb_act_quant_group128": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp]),
    "fgb_weight_quant_block128": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, ctypes.c_int, _vp]),
    "fgb_gemm_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "fgb_w8a8_block_gemm": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _vp, _vp, ctypes.c_int, _vp, ctypes.c_int,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _vp, ctypes.c_size_t, _vp]),
    "fgb_w8a8_block_gemm_noalloc": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _vp, _vp, ctypes.c_int, _vp,
                                                   ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _vp]),
    "fgb_gemm_fused_quant_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "fgb_w8a8_block_gemm_fused_quant": (ctypes.c_int, [_vp, _c_i64, _vp, _vp, ctypes.c_int, _vp, ctypes.c_int,
                                                       _c_i64, _c_i64, _c_i64, _c_i64, _vp, ctypes.c_size_t, _vp]),
    "fgb_grouped_gemm_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, ctypes.c_int32]),
    "fgb_grouped_w8a8_block_gemm": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _vp, _vp, ctypes.c_int, _vp,
                                                   ctypes.c_int32, _c_i64, _vp, ctypes.c_int, _c_i64, _c_i64,
                                                   _c_i64, _vp, ctypes.c_size_t, _vp]),
    "fgb_batched_w8a8_block_gemm": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _vp, _vp, ctypes.c_int, _vp,
                                                   ctypes.c_int32, _c_i64, _vp, ctypes.c_int, _c_i64, _c_i64,
                                                   _c_i64, _vp]),
    "fgb_check_expert_offsets": (ctypes.c_int, [_vp, ctypes.c_int32, _c_i64, _vp, _vp]),
    "fgb_act_quant_per_token": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, ctypes.c_int, _vp, _c_i64, _vp, _vp]),
    "fgb_weight_quant_per_channel": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.c_int, _vp, _vp, _vp]),
    "fgb_act_quant_static": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, ctypes.c_int, _vp, _c_i64, _vp]),
    "fgb_weight_quant_block128_ex": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp]),
    "fgb_w8a8_scaled_gemm": (ctypes.c_int, [_vp, _c_i64, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, _vp, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i64, _vp,
                                            ctypes.c_size_t, _vp]),
    "fgb_fp8_encode": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, ctypes.c_int, _vp]),
    "fgb_fp8_decode": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp]),
    "fgb_selftest_quotients": (ctypes.c_int, [_vp, _vp]),
}
EXPORTS = tuple(_SIGS)


class FGBError(ValueError):
    """A libfgb call returned a nonzero status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfgb.so (built in-tree by fine_grained_block_amd.build); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is missing: build it with `python -m fine_grained_block_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fgb_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise FGBError(fn, status, status_string(status))
