"""GPU parity: awq_linear / awq_linear_ex against the fp64 oracle."""

import numpy as np
import pytest

import workloads as wl
from gpu_common import (REL_FRO, assert_close, dev, out_to_f64, say, to_dev, to_np, torch_mod)
from oracle import (QuantConfig, bf16_bits_to_f32, dequantize, linear64, quantize_pack,
                    unpack_codes)

pytestmark = pytest.mark.gpu

GEMV, GEMM = 1, 2


def _awq():
    import bit_weight_only_quantize_amd as awq
    return awq


def _packed(W, g, chunk=4096):
    """Oracle-packed weights (row chunks bound host memory), plus GPU copies."""
    parts = [quantize_pack(W[r:r + chunk], QuantConfig(group_size=g))
             for r in range(0, W.shape[0], chunk)]
    qw, sc, zr = (np.concatenate([p[i] for p in parts]) for i in range(3))
    return qw, sc, zr, (to_dev(qw), to_dev(sc), to_dev(zr))


_PREFILL_CACHE = {}


def _x_f64(X, dt):
    return bf16_bits_to_f32(X).astype(np.float64) if dt == "bf16" else X.astype(np.float64)


def _run(X, dt, packed_dev, g, kernel, out_dtype=None):
    awq = _awq()
    Xd = to_dev(X, bf16=(dt == "bf16"))
    Y = awq.awq_linear_ex(Xd, *packed_dev, kernel=kernel, group_size=g, out_dtype=out_dtype)
    torch_mod().cuda.synchronize()
    return Y


# --- exactness pin: one-hot activations reproduce dequantized weights -------------

@pytest.mark.parametrize("kernel", [GEMV, GEMM])
@pytest.mark.parametrize("g", [64, 128])
def test_one_hot_rows_are_exact(kernel, g):
    """X = rows of the identity.  GEMV: Y[r][n] = deq[n][k_r] exactly in fp32
    (its B operand is the exact integer q - z, the scale applied in fp32).
    GEMM with fp16 activations: Y[r][n] = fp16(deq[n][k_r]) exactly, the
    dequantized weight rounded once to fp16 (its B operand)."""
    torch = torch_mod()
    N, K = 80, 512
    W = wl.gen_weight(N, K, 17)
    qw, sc, zr, pd = _packed(W, g)
    deq = dequantize(unpack_codes(qw, K), sc, zr, g)
    if kernel == GEMM:
        deq = deq.astype(np.float16).astype(np.float64)
    ks = np.arange(0, K, 37) if kernel == GEMV else np.arange(K)
    for k0 in range(0, len(ks), 16 if kernel == GEMV else len(ks)):
        sel = ks[k0:k0 + (16 if kernel == GEMV else len(ks))]
        X = np.zeros((len(sel), K), np.float16)
        X[np.arange(len(sel)), sel] = 1.0
        say("one-hot", "gemv" if kernel == GEMV else "gemm", g, len(sel))
        Y = out_to_f64(_run(X, "f16", pd, g, kernel, torch.float32))
        assert np.array_equal(Y, deq[:, sel].T)


# --- small and ragged shapes: full element-by-element comparison -------------------

RAGGED = [
    (1, 77, 320, 64, "f16"), (3, 200, 384, 128, "f16"), (16, 48, 256, 128, "bf16"),
    (5, 130, 1024, 64, "bf16"), (33, 77, 320, 64, "f16"), (77, 200, 384, 128, "f16"),
    (130, 260, 640, 64, "bf16"), (257, 129, 1152, 128, "f16"), (1, 512, 512, 128, "f16"),
    (8, 512, 512, 128, "f16"),
    # K split 8 ways with row tiles wholly or partly past M: 32-row tile at
    # M = 16 and 17, 64-row tile at M = 33
    (16, 300, 2048, 64, "f16"), (17, 300, 2048, 128, "f16"), (33, 300, 2048, 128, "bf16"),
    # GEMV with staged rows and more than 8 groups per wave (two batches in
    # flight): 8 waves per workgroup (N > 4096), K / g > 64
    (1, 5000, 8448, 128, "f16"), (2, 4200, 5120, 64, "bf16"),
    # GEMV staging of 86 and 128 KiB (16-wave workgroups, N <= 4096), and of
    # 50 and 64 KiB with 8-wave workgroups (N > 4096)
    (4, 4096, 11008, 128, "f16"), (16, 4000, 4096, 64, "bf16"),
    (5, 6000, 5120, 64, "bf16"), (8, 5000, 4096, 128, "f16"),
]


@pytest.mark.parametrize("M,N,K,g,dt", RAGGED)
def test_ragged_shapes(M, N, K, g, dt):
    torch = torch_mod()
    W = wl.gen_weight(N, K, 40 + N)
    X = wl.gen_activation(M, K, 50 + M, 51, dt)
    qw, sc, zr, pd = _packed(W, g)
    ref = linear64(_x_f64(X, dt), qw, sc, zr, g)
    kernels = [GEMM] + ([GEMV] if M <= 16 else [])
    for kern in kernels:
        say("ragged", M, N, K, g, dt, "gemv" if kern == GEMV else "gemm")
        Y32 = out_to_f64(_run(X, dt, pd, g, kern, torch.float32))
        assert_close(Y32, ref, f"{M}x{N}x{K} fp32 out")
        Y16 = out_to_f64(_run(X, dt, pd, g, kern))          # same dtype as X
        if dt == "f16":
            assert_close(Y16, ref, f"{M}x{N}x{K} 16-bit out")
        # The 16-bit output is the fp32 result rounded once.  For bf16 that
        # rounding alone (relative step 2^-8) exceeds the 1e-3 Frobenius bound,
        # so bf16 activations are held to the bound through the fp32 output.
        want = torch.from_numpy(Y32).to(torch.float16 if dt == "f16" else torch.bfloat16)
        assert np.array_equal(Y16, want.float().numpy().astype(np.float64))


# --- the 256-row tile (fp16 X, activations staged by LDS DMA) --------------------

def _takes_256_row_tile(M, N, K):
    """The plan's rule: fp16 X, K a multiple of 128, and at least 256 tiles of
    256 x 256 (so no K split)."""
    return K % 128 == 0 and ((M + 255) // 256) * ((N + 255) // 256) >= 256


@pytest.mark.parametrize("g", [64, 128])
def test_256_row_tile_one_hot_exact(g):
    """One-hot rows through the 256-row tile: Y[r][n] = fp16(deq[n][r]) exactly,
    for every row of a full 256-row tile and a ragged last column tile.  Any
    misplaced 16-byte activation chunk in the DMA-staged LDS tile breaks it."""
    torch = torch_mod()
    M = K = 256
    N = 65536 - 77
    assert _takes_256_row_tile(M, N, K)
    W = wl.gen_weight(N, K, 81)
    qw, sc, zr, pd = _packed(W, g)
    deq = dequantize(unpack_codes(qw, K), sc, zr, g).astype(np.float16).astype(np.float64)
    X = np.eye(K, dtype=np.float16)
    say("256-row tile one-hot", g, N)
    Y = out_to_f64(_run(X, "f16", pd, g, GEMM, torch.float32))
    assert np.array_equal(Y, deq.T)


@pytest.mark.parametrize("M,N,K,g,dt", [(300, 32600, 384, 128, "f16"), (1000, 16300, 256, 64, "f16"),
                                        (300, 32600, 384, 128, "bf16")])
def test_256_row_tile_ragged(M, N, K, g, dt):
    """Ragged M and N through the 256-row tile, fp32 and 16-bit output, against
    the oracle element by element.  bf16 X goes through the row prescan's
    scaled fp16 copy; some of its rows lie far outside fp16's range (up to
    ~1e8) or deep in its subnormals, and are held to the tolerance row by row
    relative to their own magnitude."""
    torch = torch_mod()
    assert _takes_256_row_tile(M, N, K)
    W = wl.gen_weight(N, K, 90 + M)
    X = wl.gen_activation(M, K, 91 + M, 92, "f16")
    if dt == "bf16":
        x = X.astype(np.float32)
        x[3] *= 3.0e6
        x[7] *= 1.0e-6
        x[260, 5] = 2.0e9            # second row tile
        x[299] *= 7.0e4              # last row
        X = wl.f32_to_bf16_bits(x)
    qw, sc, zr, pd = _packed(W, g)
    ref = linear64(_x_f64(X, dt), qw, sc, zr, g)
    say("256-row tile ragged", M, N, K, g, dt)
    Y32 = out_to_f64(_run(X, dt, pd, g, GEMM, torch.float32))
    if dt == "f16":
        assert_close(Y32, ref, f"{M}x{N}x{K} fp32 out")
    else:
        assert np.isfinite(Y32).all()
        for r in range(M):
            err = Y32[r] - ref[r]
            assert np.linalg.norm(err) <= REL_FRO * np.linalg.norm(ref[r]), f"row {r}"
            assert np.max(np.abs(err)) <= REL_FRO * np.max(np.abs(ref[r])), f"row {r}"
    Y16 = out_to_f64(_run(X, dt, pd, g, GEMM))
    if dt == "f16":
        assert_close(Y16, ref, f"{M}x{N}x{K} fp16 out")
    want = torch.from_numpy(Y32).to(torch.float16 if dt == "f16" else torch.bfloat16)
    assert np.array_equal(Y16, want.float().numpy().astype(np.float64))


def test_bf16_rows_beyond_fp16_range():
    """The GEMM runs bf16 activations in fp16 after multiplying each row by
    the power of two that brings its largest magnitude to [2^14, 2^15).  Rows
    far beyond 65504, rows of tiny values and ordinary rows all stay within
    the relative tolerance of the fp64 oracle, row by row (the max-abs bound
    is taken relative to the row's magnitude, since these rows' outputs reach
    1e7 and 1e-6)."""
    torch = torch_mod()
    M, N, K, g = 40, 300, 640, 128
    W = wl.gen_weight(N, K, 61)
    qw, sc, zr, pd = _packed(W, g)
    x = wl.gen_activation(M, K, 62, 63, "f16").astype(np.float32)
    x[3] *= 3.0e6                    # largest |x| ~ 1e8
    x[7] *= 1.0e-6                   # fp16 subnormal territory
    x[11, 5] = 2.0e9                 # one huge value in an ordinary row
    x[20] *= 7.0e4
    X = wl.f32_to_bf16_bits(x)
    ref = linear64(_x_f64(X, "bf16"), qw, sc, zr, g)
    say("bf16 wide range", M, N, K)
    Y = out_to_f64(_run(X, "bf16", pd, g, GEMM, torch.float32))
    assert np.isfinite(Y).all()
    for r in range(M):
        err = Y[r] - ref[r]
        rel = np.linalg.norm(err) / np.linalg.norm(ref[r])
        assert rel <= REL_FRO, f"row {r}: rel_fro={rel:.3e}"
        assert np.max(np.abs(err)) <= REL_FRO * np.max(np.abs(ref[r])), f"row {r}"


def test_bf16_and_split_k_calls_share_a_workspace():
    """bf16 GEMMs keep per-row activation factors in the workspace and split-K
    GEMMs their partial tiles; calls of both kinds, in turn, on one workspace
    whose initial contents are garbage (0xFF bytes: NaN as fp32) all match the
    oracle: no call depends on what an earlier one left behind."""
    torch = torch_mod()
    awq = _awq()
    # the first call sizes the library scratch so that the later ones reuse it
    shapes = [(40, 300, 640, 128), (16, 48, 256, 128), (5, 130, 1024, 64), (16, 48, 256, 128),
              (40, 300, 640, 128)]
    ws = torch.full((max(awq.awq_linear_workspace_size(64, 640, 4096, g) for g in (64, 128)),),
                    255, dtype=torch.uint8, device=dev())
    for (M, N, K, g) in shapes:
        W = wl.gen_weight(N, K, 70 + N)
        X = wl.gen_activation(M, K, 71 + M, 72, "bf16")
        qw, sc, zr, pd = _packed(W, g)
        ref = linear64(_x_f64(X, "bf16"), qw, sc, zr, g)
        say("bf16 shared workspace", M, N, K, g)
        Xd = to_dev(X, bf16=True)
        a = out_to_f64(awq.awq_linear_ex(Xd, *pd, kernel=GEMM, group_size=g,
                                         out_dtype=torch.float32))
        if M > 16:
            b = out_to_f64(awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32))
            assert_close(b, ref, f"{M}x{N}x{K} caller workspace")
        torch.cuda.synchronize()
        assert_close(a, ref, f"{M}x{N}x{K} library scratch")


def test_split_k_repeatable_and_workspace_regrowth():
    """Small-M GEMMs split K across workgroups; the partial tiles go through
    the library's per-device scratch and a second kernel sums them in split
    order.  Repeated calls give bit-identical results, and growing the
    scratch for a larger shape does not disturb a later call of the first
    shape."""
    torch = torch_mod()
    # 8 splits for the first three shapes; the fourth has 102 tiles of
    # 128 x 256, so two; the last two split 16 and 12 ways (at least 4 K
    # blocks per split beyond 8).
    shapes = [(64, 640, 4096, 128), (32, 4096, 8192, 64), (256, 1280, 2048, 128),
              (200, 13000, 512, 128), (16, 1000, 8192, 128), (40, 4000, 6144, 64)]
    outs = {}
    for rep in range(2):
        for (M, N, K, g) in shapes:
            W = wl.gen_weight(N, K, 60 + N)
            X = wl.gen_activation(M, K, 61 + M, 62, "f16")
            qw, sc, zr, pd = _packed(W, g)
            say("split-K", rep, M, N, K, g)
            Y = [out_to_f64(_run(X, "f16", pd, g, GEMM, torch.float32)) for _ in range(3)]
            assert np.array_equal(Y[0], Y[1]) and np.array_equal(Y[0], Y[2])
            if rep == 0:
                assert_close(Y[0], linear64(X.astype(np.float64), qw, sc, zr, g), f"{M}x{N}x{K}")
                outs[(M, N, K)] = Y[0]
            else:
                assert np.array_equal(Y[0], outs[(M, N, K)])


def test_caller_workspace_matches_library_scratch():
    """awq_linear_ws with a caller workspace (garbage on entry, reused) gives the
    same bits as awq_linear with the library's scratch."""
    awq = _awq()
    torch = torch_mod()
    M, N, K, g = 64, 1536, 5120, 128
    W = wl.gen_weight(N, K, 70)
    X = wl.gen_activation(M, K, 71, 72, "f16")
    qw, sc, zr, pd = _packed(W, g)
    need = awq.awq_linear_workspace_size(M, N, K, g)
    assert need > 0
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev())
    Xd = to_dev(X)
    say("workspace", M, N, K, need)
    a = awq.awq_linear(Xd, *pd, group_size=g, out_dtype=torch.float32)
    b1 = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
    b2 = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b1) and torch.equal(a, b2)
    assert_close(out_to_f64(b1), linear64(X.astype(np.float64), qw, sc, zr, g), "workspace")


def test_tiny_layer_config():
    """Tiny single layer: W 512x512, g128, X at M=1 and M=8 with 5 outlier channels."""
    torch = torch_mod()
    for case in wl.tiny_cases():
        W = case.weight()
        X = case.activation()
        qw, sc, zr, pd = _packed(W, 128)
        ref = linear64(X, qw, sc, zr, 128)
        say("tiny", case.name)
        Y = out_to_f64(_run(X, "f16", pd, 128, 0))
        assert_close(Y, ref, case.name)
        Yg = out_to_f64(_run(X, "f16", pd, 128, GEMM, torch.float32))
        Yv = out_to_f64(_run(X, "f16", pd, 128, GEMV, torch.float32))
        assert_close(Yg, ref, case.name + " gemm")
        assert_close(Yv, ref, case.name + " gemv")


# --- the decode, batched and prefill layer shapes ------------------------------------

@pytest.mark.parametrize("case", wl.gemv_cases(), ids=lambda c: c.name)
def test_decode_gemv_layers(case):
    W = case.weight()
    X = case.activation()
    qw, sc, zr, pd = _packed(W, 128)
    ref = linear64(X, qw, sc, zr, 128)
    say("gemv layer", case.name)
    assert_close(out_to_f64(_run(X, "f16", pd, 128, 0)), ref, case.name)


@pytest.mark.parametrize("case", wl.gemm_cases(), ids=lambda c: c.name)
def test_batched_gemm_layers(case):
    W = case.weight()
    X = case.activation()
    qw, sc, zr, pd = _packed(W, case.group_size)
    ref = linear64(X, qw, sc, zr, case.group_size)
    say("gemm layer", case.name)
    assert_close(out_to_f64(_run(X, "f16", pd, case.group_size, 0)), ref, case.name)


@pytest.mark.parametrize("case", wl.prefill_cases(), ids=lambda c: c.name)
def test_prefill_layers_sampled(case):
    """M=4096 prefill on 70B-class layers: every output is computed on the GPU;
    the oracle evaluates 96 sampled rows x 384 sampled columns (plus the last
    row and column) one by one."""
    torch = torch_mod()
    key = (case.K, case.N)
    if key not in _PREFILL_CACHE:
        _PREFILL_CACHE.clear()
        _PREFILL_CACHE[key] = _packed(case.weight(), 128)
    qw, sc, zr, pd = _PREFILL_CACHE[key]
    X = case.activation()
    out_dtype = torch.float16 if case.x_dtype == "f16" else torch.float32
    say("prefill layer", case.name)
    Y = _run(X, case.x_dtype, pd, 128, 0, out_dtype)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[case.M - 1], rng.choice(case.M, 96, replace=False)]))
    cols = np.unique(np.concatenate([[case.N - 1], rng.choice(case.N, 384, replace=False)]))
    ref = linear64(_x_f64(X, case.x_dtype), qw, sc, zr, 128, rows=rows, cols=cols)
    got = out_to_f64(Y)[np.ix_(rows, cols)]
    assert_close(got, ref, case.name)
    assert np.isfinite(out_to_f64(Y)).all()
    if case.x_dtype == "bf16":
        # bf16 output is the fp32 result rounded once to bf16
        Yb = _run(X, "bf16", pd, 128, 0, torch.bfloat16)
        assert torch.equal(Yb, Y.to(torch.bfloat16))


def test_gemv_and_gemm_agree_at_batch_one():
    """The GEMV scales exact q - z sums in fp32; the fp16 GEMM multiplies by
    fp16(deq) (relative error <= 2^-11 per weight).  Their difference is
    bounded per output by 2^-11 * sum_k |x_k| |deq_k| plus fp32 summation
    slack."""
    case = wl.gemv_cases(Ms=(1,))[1]
    W = case.weight()
    X = case.activation()
    torch = torch_mod()
    qw, sc, zr, pd = _packed(W, 128)
    say("gemv vs gemm", case.name)
    a = out_to_f64(_run(X, "f16", pd, 128, GEMV, torch.float32))
    b = out_to_f64(_run(X, "f16", pd, 128, GEMM, torch.float32))
    deq = dequantize(unpack_codes(qw, case.K), sc, zr, 128)
    S = np.abs(X.astype(np.float64)) @ np.abs(deq).T
    assert np.all(np.abs(a - b) <= (2.0 ** -11 + 1e-5) * S + 1e-6)


def test_empty_inputs():
    awq = _awq()
    torch = torch_mod()
    W = wl.gen_weight(32, 256, 1)
    _, _, _, pd = _packed(W, 128)
    X = torch.empty((0, 256), dtype=torch.float16, device=dev())
    Y = awq.awq_linear(X, *pd, group_size=128)
    assert Y.shape == (0, 32)
