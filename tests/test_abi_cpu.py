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
    bad_zp = binding.awq_config(4, 128, 2)
    assert _qp(c=bad_zp) == binding.AWQ_ERR_INVALID_ARG
    assert "zero_point" in lib.awq_last_error().decode()
    # the symmetric grid takes no zeros: NULL passes validation (N = 0: no launch)
    assert _qp(c=cfg(128, zero_point=False), zr=NULL, N=0) == binding.AWQ_OK
    assert _qp(zr=NULL) == binding.AWQ_ERR_INVALID_ARG      # asymmetric needs them
    assert _qp(K=192) == binding.AWQ_ERR_INVALID_ARG          # not a multiple of 128
    assert _qp(K=0) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(N=-1) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(W=NULL) == binding.AWQ_ERR_INVALID_ARG
    assert _qp(qw=ctypes.c_void_p(0x10004)) == binding.AWQ_ERR_INVALID_ARG   # misaligned
    assert _qp(s=ctypes.c_void_p(0x10008)) == binding.AWQ_ERR_INVALID_ARG
    # empty input is a successful no-op, with no HIP call
    assert _qp(N=0) == binding.AWQ_OK
    assert lib.awq_last_error().decode() == ""


def test_dequantize_validation():
    dq = lambda **k: lib.awq_dequantize(k.get("qw", FAKE), FAKE, k.get("zr", FAKE), k.get("N", 4),
                                        k.get("K", 256), k.get("c", cfg(128)), k.get("out", FAKE),
                                        k.get("dt", 2), NULL)
    assert dq(dt=1) == binding.AWQ_ERR_INVALID_ARG           # bf16 output is not offered
    assert dq(K=200) == binding.AWQ_ERR_INVALID_ARG
    assert dq(N=-1) == binding.AWQ_ERR_INVALID_ARG
    assert dq(zr=NULL) == binding.AWQ_ERR_INVALID_ARG        # asymmetric needs zeros
    assert dq(out=ctypes.c_void_p(0x10008)) == binding.AWQ_ERR_INVALID_ARG
    assert dq(N=0) == binding.AWQ_OK
    assert dq(N=0, zr=NULL, c=cfg(128, zero_point=False)) == binding.AWQ_OK


def test_fused_validation():
    P = binding.awq_linear_part
    arr = (P * 5)()
    for i in range(5):
        arr[i] = P(0x10000, 0x10000, 0x10000, 64, 0x10000)

    def call(n=2, epi=0, H=NULL, kernel=0, M=3, K=256, ws=NULL, wsb=0, xt=0):
        return lib.awq_linear_fused(FAKE, xt, arr, n, M, K, cfg(128), epi, H, 0, kernel, ws, wsb,
                                    NULL)
    assert call(n=0) == binding.AWQ_ERR_INVALID_ARG
    assert call(n=5) == binding.AWQ_ERR_INVALID_ARG
    assert call(epi=2) == binding.AWQ_ERR_INVALID_ARG
    assert call(kernel=binding.AWQ_KERNEL_BATCHED) == binding.AWQ_ERR_INVALID_ARG
    assert call(n=3, epi=1, H=FAKE) == binding.AWQ_ERR_INVALID_ARG     # the pair is 2 parts
    arr[1].N = 65
    assert call(epi=1, H=FAKE) == binding.AWQ_ERR_INVALID_ARG          # of equal N
    arr[1].N = 64
    assert call(epi=1) == binding.AWQ_ERR_INVALID_ARG                  # H is required
    assert call(K=200) == binding.AWQ_ERR_INVALID_ARG
    assert call(kernel=1, M=17) == binding.AWQ_ERR_INVALID_ARG        # GEMV serves M <= 16
    # the GEMM path of a pair needs fp32 gate/up in the workspace
    need = lib.awq_linear_fused_workspace_size(arr, 2, 64, 256, cfg(128), 0, 1, 2)
    assert need >= 2 * 64 * 64 * 4
    assert call(epi=1, H=FAKE, kernel=2, M=64, ws=FAKE, wsb=need - 1) == binding.AWQ_ERR_WORKSPACE
    assert lib.awq_linear_fused_workspace_size(arr, 2, 1, 256, cfg(128), 0, 1, 0) == 0  # GEMV
    assert call(M=0) == binding.AWQ_OK


def _lin(X=FAKE, xt=0, M=3, N=64, K=256, c=None, Y=FAKE, yt=0, kernel=0, ws=NULL, ws_bytes=0):
    return lib.awq_linear_ex(X, xt, FAKE, FAKE, FAKE, M, N, K, c or cfg(128), Y, yt, kernel, ws,
                             ws_bytes, NULL)


def test_linear_validation():
    assert _lin(xt=2) == binding.AWQ_ERR_INVALID_ARG          # fp32 activations are not W4A16
    assert _lin(yt=7) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(kernel=5) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=17, kernel=binding.AWQ_KERNEL_GEMV) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=65, kernel=binding.AWQ_KERNEL_BATCHED) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=-2) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(K=100) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(c=cfg(128, w_bit=8)) == binding.AWQ_ERR_UNSUPPORTED
    assert _lin(X=NULL) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(X=ctypes.c_void_p(0x10002)) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(Y=ctypes.c_void_p(0x10002), yt=2) == binding.AWQ_ERR_INVALID_ARG
    assert lib.awq_linear_ex(FAKE, 0, FAKE, ctypes.c_void_p(0x10001), FAKE, 3, 64, 256, cfg(128),
                             FAKE, 0, 0, NULL, 0, NULL) == binding.AWQ_ERR_INVALID_ARG  # odd scales
    assert _lin(ws=ctypes.c_void_p(0x10010), ws_bytes=1 << 20) == binding.AWQ_ERR_INVALID_ARG
    assert _lin(M=0) == binding.AWQ_OK
    assert _lin(N=0, X=NULL) == binding.AWQ_OK
    assert lib.awq_linear(FAKE, 0, FAKE, FAKE, FAKE, 3, 64, 200, cfg(128), FAKE, 0, NULL) \
        == binding.AWQ_ERR_INVALID_ARG


def _wsz(M, N, K, g=128, xd=0, kernel=0):
    return lib.awq_linear_workspace_size(M, N, K, cfg(g), xd, kernel)


def test_linear_workspace_size_and_validation():
    # one row of a 4096-wide layer runs the GEMV: no workspace
    assert _wsz(1, 4096, 4096) == 0
    # ... unless the GEMM is forced: its 16 column tiles split K
    assert _wsz(1, 4096, 4096, kernel=binding.AWQ_KERNEL_GEMM) > 0
    # a batch of 64 splits K across workgroups: fp32 partial tiles
    ws = _wsz(64, 13824, 5120)
    assert ws >= 64 * 13824 * 4
    # bf16 adds one fp32 factor per row
    assert _wsz(64, 13824, 5120, xd=1) >= ws + 64 * 4
    # the prefill shapes fill the GPU unsplit: nothing for fp16, the row
    # factors and an fp16 copy of X for bf16
    assert _wsz(4096, 28672, 8192) == 0
    assert _wsz(4096, 28672, 8192, xd=1) >= 4096 * 8192 * 2 + 4096 * 4
    # the batched-decode kernel splits K into fp32 partials [split][M][N]
    bw = _wsz(16, 13824, 5120, kernel=binding.AWQ_KERNEL_BATCHED)
    assert bw > 0 and bw % (16 * 13824 * 4) == 0
    assert _wsz(65, 13824, 5120, kernel=binding.AWQ_KERNEL_BATCHED) == 0
    assert _wsz(64, 13824, 100) == 0           # invalid K
    assert _wsz(0, 13824, 5120) == 0
    assert _wsz(64, 13824, 5120, xd=2) == 0    # fp32 activations are not W4A16
    assert _wsz(64, 13824, 5120, kernel=7) == 0

    def call(ws_ptr=FAKE, ws_bytes=ws, M=64, N=13824, K=5120):
        return lib.awq_linear_ws(FAKE, 0, FAKE, FAKE, FAKE, M, N, K, cfg(128), FAKE, 0, ws_ptr,
                                 ws_bytes, NULL)
    assert call(ws_bytes=ws - 1) == binding.AWQ_ERR_WORKSPACE
    assert "needed" in lib.awq_last_error().decode()
    assert call(ws_ptr=ctypes.c_void_p(0x10010)) == binding.AWQ_ERR_INVALID_ARG
    assert call(M=0, ws_ptr=NULL, ws_bytes=0) == binding.AWQ_OK


def test_scratch_free_calls():
    """awq_linear (and awq_linear_ex without a workspace) allocate nothing and
    use no scratch: a bf16 GEMM, which needs per-row factors in scratch
    memory, is refused before any HIP call."""
    bf = lib.awq_linear(FAKE, 1, FAKE, FAKE, FAKE, 64, 13824, 5120, cfg(128), FAKE, 2, NULL)
    assert bf == binding.AWQ_ERR_WORKSPACE
    assert "workspace" in lib.awq_last_error().decode()
    assert _lin(xt=1, M=64, N=13824, K=5120, kernel=binding.AWQ_KERNEL_GEMM) \
        == binding.AWQ_ERR_WORKSPACE
    # a workspace one byte short of the bf16 plan's is refused too
    need = _wsz(64, 13824, 5120, xd=1, kernel=binding.AWQ_KERNEL_GEMM)
    assert _lin(xt=1, M=64, N=13824, K=5120, kernel=binding.AWQ_KERNEL_GEMM,
                ws=ctypes.c_void_p(0x10000), ws_bytes=need - 1) == binding.AWQ_ERR_WORKSPACE


def test_noalloc_rejects_beyond_its_static_scratch():
    """awq_linear_noalloc refuses, before any HIP call, a call whose scratch
    exceeds its static array: bf16 activations on the GEMM path take one fp32
    factor per row, so 9 million rows need 36 MB of the 33 MiB."""
    assert binding.lib.awq_linear_noalloc(FAKE, 1, FAKE, FAKE, FAKE, 9_000_000, 4096, 4096,
                                          cfg(128), FAKE, 2, NULL) == binding.AWQ_ERR_WORKSPACE
    assert "static" in lib.awq_last_error().decode()
    assert binding.lib.awq_linear_noalloc(FAKE, 0, FAKE, FAKE, FAKE, 0, 4096, 4096, cfg(128),
                                          FAKE, 2, NULL) == binding.AWQ_OK
    assert binding.lib.awq_linear_noalloc(FAKE, 0, FAKE, FAKE, FAKE, 4, 4096, 4096, cfg(96),
                                          FAKE, 2, NULL) == binding.AWQ_ERR_UNSUPPORTED


def test_batched_split_plan():
    """The batched-decode kernel's split count (host logic, read off its
    workspace: splits x M x N fp32 partials).  The plan minimizes the busiest
    CU's groups (workgroups per CU times groups per split) plus 1.1 per split
    plus 4 for a second residency round; these are the picks that same-box
    sweeps of every split count put at (or within 0.5 us of) the fastest."""
    B = binding.AWQ_KERNEL_BATCHED

    def splits(M, N, K, g):
        w = _wsz(M, N, K, g, kernel=B)
        assert w % (M * N * 4) == 0
        return w // (M * N * 4)
    assert splits(16, 11008, 4096, 128) == 2     # 172 workgroups, one round
    assert splits(16, 13824, 5120, 128) == 4     # 432 workgroups
    assert splits(16, 5120, 13824, 128) == 12    # 480 workgroups of 9 groups
    assert splits(16, 13824, 5120, 64) == 4      # not 7: that needs a second round
    assert splits(32, 13824, 5120, 128) == 7     # 8 groups per split at most
    assert splits(8, 4096, 4096, 128) == 4
    # a range of at most 2048 / (g * ceil(M/16)) groups: 4096 / 128 = 32
    # groups at M = 64 need 8 splits even without a cost model
    assert splits(64, 4096, 4096, 128) >= 8


def test_linear_dispatch_rule():
    """The automatic kernel choice of a call with scratch (awq_linear_ws,
    awq_linear_ex with a workspace; host logic, no GPU): the batched-decode
    kernel for 2 <= M <= 32 on layers of at least 1.6e7 weights and 4096
    columns, unless the GEMV stages the activation rows (64 KiB, or 128 KiB
    when N <= 4096) and M < 8 or the layer has under 2e7 weights; else the
    GEMV wherever it stages the rows; else, unstaged, the GEMM where a GEMV
    wave would walk more than 8 groups, the GEMV up to M = 8 (12 on layers
    of at most 5e7 weights), the GEMM beyond.  The kernel is read off the
    workspace size (bf16 activations: the GEMM always needs one, the GEMV
    none, the batched kernel exactly its own)."""
    B = binding.AWQ_KERNEL_BATCHED

    def kind(M, N, K):
        a = _wsz(M, N, K, xd=1)
        if a == 0:
            return "gemv"
        if a == _wsz(M, N, K, xd=1, kernel=B):
            return "batched"
        assert a == _wsz(M, N, K, xd=1, kernel=binding.AWQ_KERNEL_GEMM)
        return "gemm"
    assert kind(2, 5120, 13824) == "gemv"       # 55 KiB of rows: staged
    assert kind(4, 5120, 13824) == "batched"    # unstaged, 7.1e7 weights
    assert kind(6, 11008, 4096) == "gemv"       # staged, M < 8
    assert kind(8, 11008, 4096) == "batched"    # staged (64 KiB), but M >= 8
    assert kind(12, 11008, 4096) == "batched"
    assert kind(8, 13824, 5120) == "batched"
    assert kind(32, 13824, 5120) == "batched"
    assert kind(33, 13824, 5120) == "gemm"      # beyond 32 rows
    assert kind(16, 4096, 4096) == "gemv"       # 128 KiB: staged, 1.7e7 weights
    assert kind(17, 4096, 4096) == "batched"    # beyond the GEMV's 16 rows
    assert kind(4, 4096, 11008) == "gemv"       # 88 KiB: staged (16-wave workgroups)
    assert kind(6, 4096, 11008) == "batched"    # 132 KiB: unstaged
    assert kind(16, 4096, 11008) == "batched"
    assert kind(8, 4000, 5120) == "gemv"        # N < 4096: staged GEMV (80 KiB, 16 waves)
    assert kind(16, 4000, 5120) == "gemm"       # N < 4096, unstaged, M > 12
    assert kind(12, 3000, 20480) == "gemm"      # N < 4096: 10 groups per GEMV wave
    assert kind(4, 6000, 4096) == "gemv"        # 2.5e7 weights: staged, M < 8
    assert kind(16, 2048, 4096) == "gemv"       # N < 4096: staged GEMV


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


def test_search_options_validation():
    O = binding.awq_search_options
    size = lambda M, N, o: lib.awq_scale_search_workspace_size_ex(M, N, 4096, cfg(128), 20,
                                                                 ctypes.byref(o))
    plain = lib.awq_scale_search_workspace_size(4096, 4096, 4096, cfg(128), 20)
    assert size(4096, 4096, O(0, 0)) == plain
    # duo adds the weights' statistic; clipping the Gram matrices (fp64)
    assert size(4096, 4096, O(1, 0)) > plain
    assert size(4096, 4096, O(0, 1)) >= plain + 32 * 128 * 128 * 8
    assert size(4096, 4096, O(2, 0)) == 0
    assert size(4096, 1 << 24, O(1, 0)) == 0         # duo: N < 2^24 rows of W
    # clipping: at most 65535 groups (K = 65536 * 128 has one too many)
    assert lib.awq_scale_search_workspace_size_ex(64, 1, 65536 * 128, cfg(128), 20,
                                                  ctypes.byref(O(0, 1))) == 0
    assert b"65535 groups" in lib.awq_last_error()
    best = ctypes.c_int32(-1)
    o = O(0, 3)
    st = lib.awq_scale_search_ex(FAKE, FAKE, 64, 64, 256, cfg(128), None, 20, ctypes.byref(o),
                                 FAKE, 1 << 40, ctypes.byref(best), None, FAKE, FAKE, FAKE, FAKE,
                                 NULL, NULL)
    assert st == binding.AWQ_ERR_INVALID_ARG and best.value == -1


def test_single_hip_runtime_in_process():
    """torch bundles a HIP runtime with the same soname; the binding must bind
    the library to that copy, never map a second runtime next to it."""
    maps = open("/proc/self/maps").read()
    runtimes = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(runtimes) == 1, runtimes


# --- the binding checks dtypes and shapes before any C call -------------------------

def _raises(exc, fn, *a, **k):
    with pytest.raises(exc) as e:
        fn(*a, **k)
    return str(e.value)


def test_binding_rejects_mismatched_tensors():
    """Wrong dtypes or shapes raise in the binding (on CPU tensors, before the
    device check and before any launch): an `out` that is too small, a
    narrower W, packed tensors of the wrong dtype or group count."""
    import torch
    M, N, K, g = 4, 64, 256, 128
    X = torch.zeros((M, K), dtype=torch.float16)
    qw = torch.zeros((N, K // 8), dtype=torch.int32)
    sc = torch.zeros((N, K // g), dtype=torch.float16)
    zr = torch.zeros((N, K // g), dtype=torch.uint8)
    lin = binding.awq_linear
    assert "out" in _raises(ValueError, lin, X, qw, sc, zr, out=torch.empty((M, N - 1), dtype=torch.float16))
    assert "out" in _raises(TypeError, lin, X, qw, sc, zr, out=torch.empty((M, N), dtype=torch.int16))
    assert "qweight" in _raises(TypeError, lin, X, qw.to(torch.int64), sc, zr)
    assert "qweight" in _raises(ValueError, lin, X, qw[:, :-1], sc, zr)
    assert "scales" in _raises(TypeError, lin, X, qw, sc.float(), zr)
    assert "scales" in _raises(ValueError, lin, X, qw, sc, zr, group_size=64)
    assert "zeros" in _raises(TypeError, lin, X, qw, sc, zr.to(torch.int8))
    assert "zeros" in _raises(ValueError, lin, X, qw, sc, zr[:-1])
    assert "X" in _raises(TypeError, lin, X.float(), qw, sc, zr)
    assert "out_dtype" in _raises(TypeError, lin, X, qw, sc, zr, out_dtype=torch.int32)
    assert "K=" in _raises(ValueError, lin, X[:, :200], qw, sc, zr)
    # everything well-formed, but on the CPU: refused for placement
    assert "GPU" in _raises(ValueError, lin, X, qw, sc, zr)
    ex = binding.awq_linear_ex
    assert "workspace" in _raises(ValueError, ex, X, qw, sc, zr, workspace="big")

    W = torch.zeros((N, K), dtype=torch.float16)
    qp = binding.awq_quantize_pack
    assert "W" in _raises(TypeError, qp, W.float())
    assert "s" in _raises(ValueError, qp, W, s=torch.ones(K - 8, dtype=torch.float32))
    assert "s" in _raises(TypeError, qp, W, s=torch.ones(K, dtype=torch.float64))
    assert "N rows" in _raises(ValueError, qp, W, out=(qw[:-1], sc[:-1], zr[:-1]))
    assert "GPU" in _raises(ValueError, qp, W)

    ss = binding.awq_scale_search
    assert "input channels" in _raises(ValueError, ss, X, W[:, :128])
    assert "W" in _raises(TypeError, ss, X, W.float())
    assert "X" in _raises(TypeError, ss, X.to(torch.bfloat16), W)
    assert "workspace" in _raises(ValueError, ss, X, W, workspace=torch.empty(16, dtype=torch.uint8))
    assert "GPU" in _raises(ValueError, ss, X, W)
