"""C-ABI tests that run without a GPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments synchronously (before any device work).

Calls with otherwise-valid arguments use fake device addresses; they must stop at the device
check, so those cases only run where no GPU is present.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgb.h")

from fine_grained_block_amd import _lib  # noqa: E402

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation returns first
ERR = dict(OK=0, NULL=-1, SHAPE=-2, STRIDE=-3, ALIGN=-4, ENUM=-5, WORKSPACE=-6, DEVICE=-7, LAUNCH=-8)


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgb_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.lib_path):
        pytest.fail("libfgb.so is not built (run `python -m fine_grained_block_amd.build`)")
    return _lib.lib()


def test_exports_every_header_symbol(L):
    funcs = header_functions()
    assert len(funcs) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fgb_[a-z0-9_]+)", out))
    missing = [f for f in funcs if f not in exported]
    assert not missing, missing
    assert set(funcs) == set(_lib.EXPORTS)
    for f in funcs:
        assert getattr(L, f) is not None


def test_version_and_status_strings(L):
    assert L.fgb_abi_version() == 1
    for name, code in ERR.items():
        s = L.fgb_status_string(code).decode()
        assert name in s
    assert L.fgb_status_string(12345).decode() == "unknown fgb status"


def _gemm(L, **kw):
    a = dict(a_q=FAKE, lda=1024, s_a=FAKE, ld_sa=256, w_q=FAKE, s_w=FAKE, fmt=0, y=FAKE, ydt=0,
             ldy=512, M=256, N=512, K=1024, ws=None, wsb=0)
    a.update(kw)
    return L.fgb_w8a8_block_gemm(a["a_q"], a["lda"], a["s_a"], a["ld_sa"], a["w_q"], a["s_w"], a["fmt"],
                                 a["y"], a["ydt"], a["ldy"], a["M"], a["N"], a["K"], a["ws"], a["wsb"], None)


def test_gemm_validation(L):
    assert _gemm(L, K=1000, lda=1008) == ERR["SHAPE"]
    assert _gemm(L, N=500) == ERR["SHAPE"]
    assert _gemm(L, M=-1) == ERR["SHAPE"]
    assert _gemm(L, M=0) == ERR["OK"]          # no-op, before any pointer or device check
    assert _gemm(L, fmt=2) == ERR["ENUM"]
    assert _gemm(L, ydt=7) == ERR["ENUM"]
    assert _gemm(L, a_q=None) == ERR["NULL"]
    assert _gemm(L, s_w=None) == ERR["NULL"]
    assert _gemm(L, lda=512) == ERR["STRIDE"]
    assert _gemm(L, ldy=256) == ERR["STRIDE"]
    assert _gemm(L, ld_sa=100) == ERR["STRIDE"]
    assert _gemm(L, a_q=FAKE + 8) == ERR["ALIGN"]
    assert _gemm(L, lda=1032) == ERR["ALIGN"]
    assert _gemm(L, ld_sa=258) == ERR["ALIGN"]
    # the decode path for 16 < M <= 64 needs a workspace when it slices K; M <= 16 and prefill do not
    need = L.fgb_gemm_workspace_bytes(40, 6144, 4096)
    assert need > 0
    assert _gemm(L, M=40, N=6144, K=4096, lda=4096, ldy=6144, ld_sa=40) == ERR["WORKSPACE"]
    assert _gemm(L, M=40, N=6144, K=4096, lda=4096, ldy=6144, ld_sa=40, ws=FAKE, wsb=need - 1) == ERR["WORKSPACE"]
    # at most 32 rows with 32-63 K-blocks: workgroups of 2 or 4 waves over the whole K, no slices
    assert L.fgb_gemm_workspace_bytes(32, 6144, 4096) == 0
    assert L.fgb_gemm_workspace_bytes(17, 10240, 5248) == 0
    assert L.fgb_gemm_workspace_bytes(32, 4096, 8192) > 0
    # weights of at most 16 MiB take the one-launch ring kernel at 16 < M <= 64
    assert L.fgb_gemm_workspace_bytes(64, 4096, 4096) == 0
    assert L.fgb_gemm_workspace_bytes(16, 4096, 4096) == 0
    assert L.fgb_gemm_workspace_bytes(1, 4096, 4096) == 0
    # unsliced 16 < M <= 64 shapes (224 workgroups of 128 weight rows) need none either
    assert L.fgb_gemm_workspace_bytes(64, 28672, 4096) == 0
    # 65-128 rows with K <= 8192: the shared-ring decode kernel with 128 activation rows, K-sliced
    # by the same rule as at 33-64 rows (the per-wave ring kernel of 4096x4096 stops at 64 rows);
    # longer rows take the prefill tiles
    assert L.fgb_gemm_workspace_bytes(128, 4096, 4096) == 4 * 128 * 4096 * 4     # 32 blocks of 128 rows
    assert L.fgb_gemm_workspace_bytes(100, 28672, 4096) == 0                     # 224 weight blocks
    assert L.fgb_gemm_workspace_bytes(65, 4096, 14336) == 16 * 65 * 4096 * 4     # prefill: 16 tiles, 16 slices
    # the boundaries of the decode route: K = 8192 (64 blocks) and 128 rows
    assert L.fgb_gemm_workspace_bytes(100, 4096, 8192) == 7 * 100 * 4096 * 4     # decode, 7 slices of 10
    assert L.fgb_gemm_workspace_bytes(100, 4096, 8320) == 13 * 100 * 4096 * 4    # prefill, 13 slices of 5
    assert L.fgb_gemm_workspace_bytes(128, 4096, 8192) == 7 * 128 * 4096 * 4     # decode
    assert L.fgb_gemm_workspace_bytes(129, 4096, 8192) == 8 * 129 * 4096 * 4     # prefill, 32 tiles
    # prefill (M > 128): K is sliced when the 256x128 tiles (128x128 when N % 256 != 0) would
    # occupy fewer than half of the 256 CUs (the count the query assumes without a device):
    # S = min(CUs / tiles, K-blocks / 4, 16, 32 MiB / (M*N*4)), then S * M * N float32 partials
    MiB = 1 << 20
    assert L.fgb_gemm_workspace_bytes(256, 4096, 4096) == 8 * 256 * 4096 * 4      # 32 tiles, 32 K-blocks
    assert L.fgb_gemm_workspace_bytes(256, 4096, 14336) == 8 * 256 * 4096 * 4     # capped at 32 MiB
    assert L.fgb_gemm_workspace_bytes(129, 28672, 4096) == 0                      # 224 tiles
    assert L.fgb_gemm_workspace_bytes(192, 14336, 4096) == 2 * 192 * 14336 * 4    # 112 tiles, 16-block slices
    assert L.fgb_gemm_workspace_bytes(192, 12288, 1536) == 0                      # 96 tiles, 6-block slices
    assert L.fgb_gemm_workspace_bytes(384, 7168, 18432) == 3 * 384 * 7168 * 4     # 84 tiles, 48-block slices
    assert L.fgb_gemm_workspace_bytes(200, 1152, 1024) == 2 * 200 * 1152 * 4      # 128x128 tiles, 8 K-blocks
    assert L.fgb_gemm_workspace_bytes(4096, 4096, 4096) == 0                      # 512 tiles
    assert L.fgb_gemm_workspace_bytes(1024, 28672, 4096) == 0                     # partials above 32 MiB
    assert L.fgb_gemm_workspace_bytes(256, 4096, 512) == 0                        # 4 K-blocks: one slice
    for M, N, K in [(130, 512, 2048), (256, 4096, 14336), (512, 4096, 14336), (300, 1024, 1024),
                    (128, 7168, 18432), (65, 49024, 128 * 8)]:
        assert L.fgb_gemm_workspace_bytes(M, N, K) <= 32 * MiB
    for M in (128, 256):
        need = L.fgb_gemm_workspace_bytes(M, 4096, 4096)
        assert _gemm(L, M=M, N=4096, K=4096, lda=4096, ldy=4096, ld_sa=M) == ERR["WORKSPACE"]
        assert _gemm(L, M=M, N=4096, K=4096, lda=4096, ldy=4096, ld_sa=M, ws=FAKE, wsb=need - 16) == ERR["WORKSPACE"]


def test_fused_quant_workspace(L):
    """The fused-quantization decode call needs a workspace exactly where it quantizes into one
    (one launch only for M <= 4 with K >= 4096 or M <= 8 with weights of at most 16 MiB); sizes
    are checked first."""
    q = L.fgb_gemm_fused_quant_workspace_bytes
    for M, N, K in [(1, 28672, 4096), (4, 7168, 18432), (8, 4096, 4096), (8, 1024, 2048)]:
        assert q(M, N, K) == 0
    for M, N, K in [(5, 28672, 4096), (1, 24576, 1536), (8, 6144, 4096), (9, 4096, 4096), (64, 4096, 4096)]:
        # at least the codes [M, K] and the scales [K/128, M] float32
        assert q(M, N, K) >= M * K + 4 * M * (K // 128)
    assert q(65, 4096, 4096) == 0 and q(16, 4000, 4096) == 0
    f = L.fgb_w8a8_block_gemm_fused_quant
    need = q(32, 4096, 4096)
    args = lambda ws, wsb, M=32: (FAKE, 4096, FAKE, FAKE, 0, FAKE, 0, 4096, M, 4096, 4096, ws, wsb, None)
    assert f(*args(None, 0)) == ERR["WORKSPACE"]
    assert f(*args(FAKE, need - 1)) == ERR["WORKSPACE"]
    assert f(*args(FAKE + 8, need)) == ERR["ALIGN"]
    assert f(*args(None, 0, M=65)) == ERR["SHAPE"]


def test_check_expert_offsets_validation(L):
    """The offsets check validates its arguments before any device work."""
    assert L.fgb_check_expert_offsets(FAKE, 0, 10, FAKE, None) == ERR["SHAPE"]
    assert L.fgb_check_expert_offsets(FAKE, 65536, 10, FAKE, None) == ERR["SHAPE"]
    assert L.fgb_check_expert_offsets(FAKE, 4, -1, FAKE, None) == ERR["SHAPE"]
    assert L.fgb_check_expert_offsets(None, 4, 10, FAKE, None) == ERR["NULL"]
    assert L.fgb_check_expert_offsets(FAKE, 4, 10, None, None) == ERR["NULL"]
    assert L.fgb_check_expert_offsets(FAKE + 2, 4, 10, FAKE, None) == ERR["ALIGN"]
    assert L.fgb_check_expert_offsets(FAKE, 4, 10, FAKE + 1, None) == ERR["ALIGN"]


@pytest.mark.skipif(_has_gpu(), reason="fake pointers must not reach a real device")
def test_valid_arguments_stop_at_device_check(L):
    assert _gemm(L, ws=FAKE, wsb=L.fgb_gemm_workspace_bytes(256, 512, 1024)) == ERR["DEVICE"]  # K-sliced prefill
    assert _gemm(L, M=512, N=512, K=512, lda=512, ld_sa=512) == ERR["DEVICE"]  # unsliced prefill, no workspace
    assert L.fgb_act_quant_group128(FAKE, 64, 1024, 1024, FAKE, 1024, FAKE, 64, None) == ERR["DEVICE"]
    assert L.fgb_fp8_decode(FAKE, FAKE, 256, 0, None) == ERR["DEVICE"]


def test_act_quant_validation(L):
    f = L.fgb_act_quant_group128
    assert f(FAKE, 64, 1000, 1000, FAKE, 1008, FAKE, 64, None) == ERR["SHAPE"]
    assert f(FAKE, 0, 1024, 1024, FAKE, 1024, FAKE, 64, None) == ERR["OK"]
    assert f(None, 64, 1024, 1024, FAKE, 1024, FAKE, 64, None) == ERR["NULL"]
    assert f(FAKE, 64, 1024, 512, FAKE, 1024, FAKE, 64, None) == ERR["STRIDE"]
    assert f(FAKE, 64, 1024, 1024, FAKE, 1024, FAKE, 32, None) == ERR["STRIDE"]
    assert f(FAKE, 64, 1024, 1028, FAKE, 1024, FAKE, 64, None) == ERR["ALIGN"]
    assert f(FAKE, 64, 1024, 1024, FAKE, 1024, FAKE, 66, None) == ERR["ALIGN"]
    assert f(FAKE + 2, 64, 1024, 1024, FAKE, 1024, FAKE, 64, None) == ERR["ALIGN"]


def test_weight_quant_and_grouped_validation(L):
    w = L.fgb_weight_quant_block128
    assert w(FAKE, 130, 128, FAKE, FAKE, 0, None) == ERR["SHAPE"]
    assert w(FAKE, 128, 128, FAKE, FAKE, 5, None) == ERR["ENUM"]
    assert w(None, 128, 128, FAKE, FAKE, 0, None) == ERR["NULL"]
    g = L.fgb_grouped_w8a8_block_gemm
    args = [FAKE, 1024, FAKE, 256, FAKE, FAKE, 0, FAKE, 4, 256, FAKE, 0, 512, 512, 1024, None, 0, None]
    bad = list(args); bad[8] = 0
    assert g(*bad) == ERR["SHAPE"]
    bad = list(args); bad[7] = None
    assert g(*bad) == ERR["NULL"]
    bad = list(args); bad[7] = FAKE + 2
    assert g(*bad) == ERR["ALIGN"]
    bad = list(args); bad[9] = 0
    assert g(*bad) == ERR["OK"]
    bad = list(args); bad[13] = 100
    assert g(*bad) == ERR["SHAPE"]


def test_codec_validation(L):
    assert L.fgb_fp8_encode(FAKE, FAKE, 16, 9, 1, None) == ERR["ENUM"]
    assert L.fgb_fp8_decode(FAKE, FAKE, 16, 3, None) == ERR["ENUM"]
    assert L.fgb_fp8_encode(FAKE, FAKE, -1, 0, 1, None) == ERR["SHAPE"]
    assert L.fgb_fp8_encode(None, FAKE, 16, 0, 1, None) == ERR["NULL"]
    assert L.fgb_fp8_decode(FAKE, FAKE + 1, 16, 0, None) == ERR["ALIGN"]
    assert L.fgb_fp8_encode(FAKE, FAKE, 0, 0, 1, None) == ERR["OK"]


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()
