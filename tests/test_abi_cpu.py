"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq355.h")

binding = pytest.importorskip("bit_weight_only_quantize_amd.binding",
                              reason="libawq355.so not built")
lib = binding.lib
cfg = binding.config


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings_and_version():
    for code in range(6):
        s = lib.awq_status_string(code).decode()
        assert s.startswith("AWQ_")
    assert lib.awq_status_string(99).decode() == "unknown awq_status"
    assert "gfx950" in lib.awq_version().decode()


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: calls fail validation first
NULL = ctypes.c_void_p(0)


def _qp(W=FAKE, N=4, K=256, c=None, s=NULL, qw=FAKE, sc=FAKE, zr=FAKE, nf=NULL):
    return lib.awq_quantize_pack(W, N, K, c or cfg(128), s, qw, sc, zr, nf, NULL)


def test_quantize_pack_validation():
    assert _qp(c=cfg(128, w_bit=3)) == binding.AWQ_ERR_UNSUPPORTED
    assert "w_bit" in lib.awq_last_error().decode()
    assert _qp(c=cfg(96)) == binding.AWQ_ERR_UNSUPPORTED
    assert _qp(c=cfg(128, zero_point=False)) == binding.AWQ_ERR_UNSUPPORTED
    assert _qp(K=192) == binding.AWQ_ERR_INVALID_ARG          # not a multiple of 128
    assert _qp(K=0) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(N=-1) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(W=NULL) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(qw=ctypes.c_void_p(0x10004)) == binding.AWQ_ERR_INVALID_ARG   # misaligned
    assert _qp(s=ctypes.c_void_p(0x10008)) == binding.AWQ_ERR_INVALID_ARG
    # empty input is a successful no-op, with no HIP call
    assert _qp(N=0) == binding.AWQ_OK
    assert lib.awq_last_error().decode() == ""


def _lin(X=FAKE, xt=0, M=3, N=64, K=256, c=None, Y=FAKE, yt=0, kernel=0):
    return lib.awq_linear_ex(X, xt, FAKE, FAKE, FAKE, M, N, K, c or cfg(128), Y, yt, kernel, NULL)


def test_linear_validation():
    assert _lin(xt=2) == binding.AWQ_ERR_INVALID_ARG          # fp32 activations are not W4A16
    assert _lin(yt=7) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(kernel=5) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=17, kernel=binding.AWQ_KERNEL_GEMV) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=-2) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(K=100) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(c=cfg(128, w_bit=8)) == binding.AWQ_ERR_UNSUPPORTED
    assert _lin(X=NULL) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(X=ctypes.c_void_p(0x10002)) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(Y=ctypes.c_void_p(0x10002), yt=2) == binding.AWQ_ERR_INVALID_ARG
    assert lib.awq_linear_ex(FAKE, 0, FAKE, ctypes.c_void_p(0x10001), FAKE, 3, 64, 256, cfg(128),
                             FAKE, 0, 0, NULL) == binding.AWQ_ERR_INVALID_ARG   # odd scales
    assert _lin(M=0) == binding.AWQ_OK
    assert _lin(N=0, X=NULL) == binding.AWQ_OK
    assert lib.awq_linear(FAKE, 0, FAKE, FAKE, FAKE, 3, 64, 200, cfg(128), FAKE, 0, NULL) \
        == binding.AWQ_ERR_INVALID_ARG


def test_linear_workspace_size_and_validation():
    # one row of a 4096-wide layer runs the GEMV: no workspace
    assert lib.awq_linear_workspace_size(1, 4096, 4096, cfg(128)) == 0
    # a batch of 64 splits K across workgroups: fp32 partial tiles
    ws = lib.awq_linear_workspace_size(64, 13824, 5120, cfg(128))
    assert ws >= 64 * 13824 * 4
    assert lib.awq_linear_workspace_size(64, 13824, 100, cfg(128)) == 0     # invalid K
    assert lib.awq_linear_workspace_size(0, 13824, 5120, cfg(128)) == 0

    def call(ws_ptr=FAKE, ws_bytes=ws, M=64, N=13824, K=5120):
        return lib.awq_linear_ws(FAKE, 0, FAKE, FAKE, FAKE, M, N, K, cfg(128), FAKE, 0, ws_ptr,
                                 ws_bytes, NULL)
    assert call(ws_bytes=ws - 1) == binding.AWQ_ERR_WORKSPACE
    assert call(ws_ptr=NULL) == binding.AWQ_ERR_INVALID_ARG
    assert call(ws_ptr=ctypes.c_void_p(0x10010)) == binding.AWQ_ERR_INVALID_ARG
    assert call(M=0, ws_ptr=NULL, ws_bytes=0) == binding.AWQ_OK


def test_linear_dispatch_rule():
    """awq_linear's GEMV/GEMM choice (host logic, no GPU): the GEMV, which
    needs no workspace, wherever its activation rows fit in LDS (64 KiB, or
    128 KiB when N <= 4096); unstaged, the GEMM (split K, so a workspace)
    where a GEMV wave would walk more than 8 groups, else the GEMV up to
    M = 8, or 12 for layers of at most 5e7 weights."""
    ws = lambda M, N, K: lib.awq_linear_workspace_size(M, N, K, cfg(128))
    assert ws(2, 5120, 13824) == 0          # 55 KiB of rows: staged
    assert ws(4, 5120, 13824) > 0           # unstaged, 108 groups over 8 waves
    assert ws(8, 11008, 4096) == 0          # 64 KiB: staged
    assert ws(12, 11008, 4096) == 0         # unstaged, 4.5e7 weights, M <= 12
    assert ws(16, 11008, 4096) > 0          # unstaged, 4.5e7 weights, M > 12
    assert ws(12, 13824, 5120) > 0          # unstaged, 7.1e7 weights, M > 8
    assert ws(8, 13824, 5120) == 0          # unstaged, M <= 8, 5 groups per wave
    assert ws(16, 4096, 4096) == 0          # 128 KiB: staged (16-wave workgroups)
    assert ws(6, 4096, 11008) == 0          # unstaged, 4.5e7 weights
    assert ws(17, 4096, 4096) > 0           # beyond the GEMV's 16 rows


def test_search_workspace_and_validation():
    ws = lib.awq_scale_search_workspace_size(4096, 4096, 4096, cfg(128), 20)
    # dominated by the fp32 reference output and the scaled activation copy
    assert 4096 * 4096 * 4 + 4096 * 4096 * 2 < ws < 4096 * 4096 * 7
    assert lib.awq_scale_search_workspace_size(0, 4096, 4096, cfg(128), 20) == 0
    assert lib.awq_scale_search_workspace_size(16, 16, 4096, cfg(128), 65) == 0
    assert lib.awq_scale_search_workspace_size(16, 16, 100, cfg(128), 20) == 0
    best = ctypes.c_int32(-1)

    def call(M=64, N=64, K=256, alphas=None, n_alpha=20, ws_ptr=FAKE, ws_bytes=1 << 40):
        return lib.awq_scale_search(FAKE, FAKE, M, N, K, cfg(128), alphas, n_alpha, ws_ptr,
                                    ws_bytes, ctypes.byref(best), None, FAKE, FAKE, FAKE, FAKE,
                                    NULL)

    assert call(n_alpha=10) == binding.AWQ_ERR_INVALID_ARG      # NULL alphas means 20 points
    bad = (ctypes.c_double * 2)(0.5, 1.5)
    assert call(alphas=ctypes.cast(bad, ctypes.POINTER(ctypes.c_double)), n_alpha=2) \
        == binding.AWQ_ERR_INVALID_ARG
    assert call(ws_bytes=100) == binding.AWQ_ERR_WORKSPACE
    assert call(ws_ptr=ctypes.c_void_p(0x10010)) == binding.AWQ_ERR_INVALID_ARG  # not 256-aligned
    assert call(M=0) == binding.AWQ_ERR_INVALID_ARG
    assert best.value == -1      # nothing written on error


def test_single_hip_runtime_in_process():
    """torch bundles a HIP runtime with the same soname; the binding must bind
    the library to that copy, never map a second runtime next to it."""
    maps = open("/proc/self/maps").read()
    runtimes = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(runtimes) == 1, runtimes
