"""GPU parity: awq_linear / awq_linear_ex against the fp64 oracle."""

import numpy as np
import pytest

import workloads as wl
from gpu_common import (REL_FRO, assert_close, dev, out_to_f64, say, to_dev, to_np, torch_mod)
from oracle import (QuantConfig, bf16_bits_to_f32, dequantize, gate_up_silu64, linear64,
                    quantize_pack, unpack_codes)

pytestmark = pytest.mark.gpu

GEMV, GEMM, BATCHED = 1, 2, 3


def _awq():
    import bit_weight_only_quantize_amd as awq
    return awq


def _packed(W, g, chunk=4096, zero_point=True):
    """Oracle-packed weights (row chunks bound host memory), plus GPU copies;
    zeros are None for the symmetric grid."""
    parts = [quantize_pack(W[r:r + chunk], QuantConfig(group_size=g, zero_point=zero_point))
             for r in range(0, W.shape[0], chunk)]
    qw, sc = (np.concatenate([p[i] for p in parts]) for i in range(2))
    zr = np.concatenate([p[2] for p in parts]) if zero_point else None
    return qw, sc, zr, (to_dev(qw), to_dev(sc), None if zr is None else to_dev(zr))


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

@pytest.mark.parametrize("path", ["gemv", "gemm32", "gemm_large", "batched"])
@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_one_hot_rows_are_exact(path, g, dt):
    """X = rows of the identity.  GEMV, the batched-decode kernel (also
    through its split-K partials: every other group contributes an exact 0)
    and the GEMM's 32-row tile (batches of up to 32 rows): Y[r][n] =
    deq[n][k_r] exactly in fp32 (their B operand is the exact integer q - z,
    the scale applied to fp32 sums).  Larger GEMM tiles: Y[r][n] =
    fp16(deq[n][k_r]) exactly, the dequantized weight rounded once to fp16
    (their B operand)."""
    torch = torch_mod()
    N, K = 80, 512
    W = wl.gen_weight(N, K, 17)
    qw, sc, zr, pd = _packed(W, g)
    deq = dequantize(unpack_codes(qw, K), sc, zr, g)
    if path == "gemm_large":
        deq = deq.astype(np.float16).astype(np.float64)
    rows = {"gemv": 16, "gemm32": 32, "gemm_large": K, "batched": 64}[path]
    kernel = {"gemv": GEMV, "batched": BATCHED}.get(path, GEMM)
    ks = np.arange(0, K, 37) if path == "gemv" else np.arange(K)
    for k0 in range(0, len(ks), rows):
        sel = ks[k0:k0 + rows]
        X = np.zeros((len(sel), K), np.float32)
        X[np.arange(len(sel)), sel] = 1.0
        X = wl.f32_to_bf16_bits(X) if dt == "bf16" else X.astype(np.float16)
        say("one-hot", path, g, dt, len(sel))
        Y = out_to_f64(_run(X, dt, pd, g, kernel, torch.float32))
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
    # GEMV with unstaged rows (over 64 KiB) on 8-wave workgroups: two groups
    # per batch, the pipelined loop and its one- and two-batch tails
    (12, 4200, 4096, 128, "f16"), (16, 4100, 5120, 64, "bf16"),
    # batched-decode kernel at g = 64, whose weight loads are refilled two
    # groups at a time: an odd group count (45) and a partial column block,
    # with one and two row tiles
    (9, 4200, 2880, 64, "f16"), (24, 4200, 2880, 64, "bf16"),
]


@pytest.mark.parametrize("M,N,K,g,dt", RAGGED)
def test_ragged_shapes(M, N, K, g, dt):
    torch = torch_mod()
    W = wl.gen_weight(N, K, 40 + N)
    X = wl.gen_activation(M, K, 50 + M, 51, dt)
    qw, sc, zr, pd = _packed(W, g)
    ref = linear64(_x_f64(X, dt), qw, sc, zr, g)
    kernels = [GEMM] + ([GEMV] if M <= 16 else []) + ([BATCHED] if M <= 64 else [])
    for kern in kernels:
        say("ragged", M, N, K, g, dt, {GEMV: "gemv", GEMM: "gemm", BATCHED: "batched"}[kern])
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
    shapes = [(40, 300, 640, 128), (16, 48, 256, 128), (5, 130, 1024, 64), (16, 48, 256, 128),
              (40, 300, 640, 128)]
    ws = torch.full((max(awq.awq_linear_workspace_size(M, N, K, g, torch.bfloat16)
                         for (M, N, K, g) in shapes),),
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


def test_split_k_repeatable():
    """Small-M GEMMs split K across workgroups; the partial tiles go through
    the workspace and a second kernel sums them in split order.  Repeated
    calls give bit-identical results, also after calls of other shapes."""
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


def test_caller_workspace_and_scratch_free_calls():
    """awq_linear_ws with a caller workspace (garbage on entry, reused) gives
    the same bits as awq_linear_ex with a workspace of its own.  awq_linear,
    which uses no scratch, runs the same layer without splitting K: within
    tolerance of the oracle, and a bf16 GEMM there is refused with
    AWQ_ERR_WORKSPACE."""
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
    a = awq.awq_linear_ex(Xd, *pd, group_size=g, out_dtype=torch.float32)
    b1 = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
    b2 = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
    c = awq.awq_linear(Xd, *pd, group_size=g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b1) and torch.equal(a, b2)
    ref = linear64(X.astype(np.float64), qw, sc, zr, g)
    assert_close(out_to_f64(b1), ref, "workspace")
    assert_close(out_to_f64(c), ref, "scratch-free")
    Xb = to_dev(wl.gen_activation(M, K, 73, 72, "bf16"), bf16=True)
    with pytest.raises(awq.AwqError) as e:
        awq.awq_linear(Xb, *pd, group_size=g, out_dtype=torch.float32)
    assert e.value.status == 3      # AWQ_ERR_WORKSPACE


def test_graph_capture_on_first_use():
    """A split-K call and a bf16 call, each captured in a HIP graph the first
    time its shape is used (the binding takes the workspace from torch's
    graph pool; the library allocates nothing), replay bit-identical to eager
    awq_linear_ws, with eager work and synchronization between replays."""
    awq = _awq()
    torch = torch_mod()
    for (M, N, K, g, dt) in [(24, 3000, 4096, 128, "f16"), (40, 2600, 3072, 64, "bf16"),
                             (14, 5000, 7168, 128, "f16")]:
        W = wl.gen_weight(N, K, 110 + M)
        X = wl.gen_activation(M, K, 111 + M, 112, dt)
        qw, sc, zr, pd = _packed(W, g)
        Xd = to_dev(X, bf16=(dt == "bf16"))
        need = awq.awq_linear_workspace_size(M, N, K, g, Xd.dtype)
        assert need > 0
        say("graph capture", M, N, K, g, dt)
        out = torch.empty((M, N), dtype=torch.float32, device=dev())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            awq.awq_linear_ex(Xd, *pd, group_size=g, out=out)
        ws = torch.full((need,), 255, dtype=torch.uint8, device=dev())
        eager = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(out_to_f64(eager), linear64(_x_f64(X, dt), qw, sc, zr, g), "eager")
        for rep in range(4):
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
            # eager work of another shape on the same workspace in between
            awq.awq_linear_ws(Xd[:M // 2].contiguous(), *pd, ws, group_size=g,
                              out_dtype=torch.float32)
            torch.cuda.synchronize()
        del graph


# --- activations with a non-zero mean -----------------------------------------------

@pytest.mark.parametrize("kind", wl.SHIFTED_KINDS)
@pytest.mark.parametrize("M,K,N,dt", [(1, 4096, 11008, "f16"), (4, 11008, 4096, "f16"),
                                      (4, 11008, 4096, "bf16")])
def test_nonzero_mean_activations(kind, M, K, N, dt):
    """|N(0,1)|, N(3,1) and N(0,1)+40 activations on the decode layers (with
    their per-row weight magnitudes), fp32 output: outputs reach several
    hundred, so any rounding of dequantized weights or cancellation of large
    biased sums would show in the max-abs error.  The GEMV and the GEMM's
    32-row tile multiply by the exact integers q - z and stay within the
    tolerance of the fp64 oracle."""
    torch = torch_mod()
    case = [c for c in wl.gemv_cases(Ms=(1,)) if c.K == K and c.N == N][0]
    W = case.weight()
    X = wl.gen_activation_shifted(M, K, 130 + M, kind, dt)
    qw, sc, zr, pd = _packed(W, 128)
    ref = linear64(_x_f64(X, dt), qw, sc, zr, 128)
    for kern in (GEMV, GEMM):
        say("non-zero mean", kind, M, K, N, dt, "gemv" if kern == GEMV else "gemm")
        Y = out_to_f64(_run(X, dt, pd, 128, kern, torch.float32))
        rel, mx = assert_close(Y, ref, f"{kind} {M}x{K}x{N} {dt} kernel {kern}")
        say("  rel_fro %.2e max_abs %.2e max|Y| %.1f" % (rel, mx, np.abs(ref).max()))


@pytest.mark.parametrize("M", [64, 300])
def test_larger_tiles_error_bound_nonzero_mean(M):
    """The GEMM's 64- and 128-row tiles round each dequantized weight once to
    fp16.  On N(0,1)+40 activations (outputs in the hundreds) every output
    stays within the bound stated for them, 2^-11 * sum_k |x_k * w_k| plus
    fp32 summation slack, and the relative Frobenius error within 1e-3."""
    torch = torch_mod()
    K, N = 4096, 3000
    W = wl.gen_weight(N, K, 140)
    X = wl.gen_activation_shifted(M, K, 141, "mean40")
    qw, sc, zr, pd = _packed(W, 128)
    deq = dequantize(unpack_codes(qw, K), sc, zr, 128)
    ref = X.astype(np.float64) @ deq.T
    S = np.abs(X.astype(np.float64)) @ np.abs(deq).T
    say("larger tiles bound", M)
    Y = out_to_f64(_run(X, "f16", pd, 128, GEMM, torch.float32))
    err = np.abs(Y - ref)
    assert np.all(err <= (2.0 ** -11 + 2.0 ** -20) * S)
    assert np.linalg.norm(Y - ref) <= REL_FRO * np.linalg.norm(ref)


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


@pytest.mark.parametrize("case", wl.gemm_cases(Ms=(16, 32, 64)), ids=lambda c: c.name)
def test_batched_decode_kernel_layers(case):
    """The batched-decode kernel on the 13B-class layers at M = 16, 32 and 64
    (one, two and four row tiles),
    K split (partials summed in split order), against the oracle; repeated
    calls are bit-identical.  Without a workspace these K need more than one
    split, and the call says so (AWQ_ERR_WORKSPACE) rather than running."""
    torch = torch_mod()
    awq = _awq()
    W = case.weight()
    X = case.activation()
    qw, sc, zr, pd = _packed(W, case.group_size)
    ref = linear64(X, qw, sc, zr, case.group_size)
    Xd = to_dev(X)
    say("batched kernel layer", case.name)
    a = awq.awq_linear_ex(Xd, *pd, kernel=BATCHED, group_size=case.group_size,
                          out_dtype=torch.float32)
    b = awq.awq_linear_ex(Xd, *pd, kernel=BATCHED, group_size=case.group_size,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert_close(out_to_f64(a), ref, case.name)
    with pytest.raises(awq.AwqError) as e:
        awq.awq_linear_ex(Xd, *pd, kernel=BATCHED, group_size=case.group_size, workspace=None)
    assert e.value.status == 3      # AWQ_ERR_WORKSPACE


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
    """At batch one both the GEMV and the GEMM (its 32-row tile) scale exact
    q - z sums in fp32: they differ only in the order of fp32 additions,
    far inside 2^-11 * sum_k |x_k| |deq_k| (the bound of the larger GEMM
    tiles, which round dequantized weights to fp16)."""
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
    assert np.all(np.abs(a - b) <= 2.0 ** -18 * S + 1e-6)


def test_empty_inputs():
    awq = _awq()
    torch = torch_mod()
    W = wl.gen_weight(32, 256, 1)
    _, _, _, pd = _packed(W, 128)
    X = torch.empty((0, 256), dtype=torch.float16, device=dev())
    Y = awq.awq_linear(X, *pd, group_size=128)
    assert Y.shape == (0, 32)


# --- the symmetric grid (zero_point=False: no zero points, zero code 8) ---------------

@pytest.mark.parametrize("path", ["gemv", "gemm32", "gemm_large"])
def test_symmetric_one_hot_rows_are_exact(path):
    torch = torch_mod()
    N, K, g = 80, 512, 128
    W = wl.gen_weight(N, K, 18)
    qw, sc, zr, pd = _packed(W, g, zero_point=False)
    assert zr is None and pd[2] is None
    deq = dequantize(unpack_codes(qw, K), sc, None, g)
    if path == "gemm_large":
        deq = deq.astype(np.float16).astype(np.float64)
    rows = {"gemv": 16, "gemm32": 32, "gemm_large": K}[path]
    for k0 in range(0, K, rows):
        sel = np.arange(k0, min(K, k0 + rows))
        X = np.zeros((len(sel), K), np.float16)
        X[np.arange(len(sel)), sel] = 1.0
        say("symmetric one-hot", path, len(sel))
        Y = out_to_f64(_run(X, "f16", pd, g, GEMV if path == "gemv" else GEMM, torch.float32))
        assert np.array_equal(Y, deq[:, sel].T)


@pytest.mark.parametrize("case", wl.gemv_cases(), ids=lambda c: c.name)
def test_symmetric_decode_layers(case):
    """The 7B-class decode layers without zero points at M = 1 and 4: the
    automatic choice (GEMV) and the GEMM, against the fp64 oracle."""
    torch = torch_mod()
    W = case.weight()
    X = case.activation()
    qw, sc, zr, pd = _packed(W, 128, zero_point=False)
    ref = linear64(X, qw, sc, None, 128)
    for kern in (0, GEMM):
        say("symmetric gemv layer", case.name, kern)
        assert_close(out_to_f64(_run(X, "f16", pd, 128, kern)), ref, case.name)
        assert_close(out_to_f64(_run(X, "f16", pd, 128, kern, torch.float32)), ref, case.name)


@pytest.mark.parametrize("case", [c for c in wl.gemm_cases() if c.M in (16, 256)],
                         ids=lambda c: c.name)
def test_symmetric_batched_layers(case):
    W = case.weight()
    X = case.activation()
    qw, sc, zr, pd = _packed(W, case.group_size, zero_point=False)
    ref = linear64(X, qw, sc, None, case.group_size)
    say("symmetric gemm layer", case.name)
    assert_close(out_to_f64(_run(X, "f16", pd, case.group_size, 0)), ref, case.name)


@pytest.mark.parametrize("M,N,K,g,dt", [(5, 130, 1024, 64, "bf16"), (33, 300, 2048, 128, "bf16"),
                                        (77, 200, 384, 128, "f16"), (300, 32600, 384, 128, "bf16")])
def test_symmetric_ragged(M, N, K, g, dt):
    """Ragged symmetric layers through the GEMV, the split-K tiles and the
    256-row tile, fp16 and bf16 activations, fp32 output; awq_linear_noalloc
    gives the same bits as the workspace call."""
    torch = torch_mod()
    awq = _awq()
    W = wl.gen_weight(N, K, 180 + N)
    X = wl.gen_activation(M, K, 181 + M, 182, dt)
    qw, sc, zr, pd = _packed(W, g, zero_point=False)
    ref = linear64(_x_f64(X, dt), qw, sc, None, g)
    for kern in [GEMM] + ([GEMV] if M <= 16 else []) + ([BATCHED] if M <= 64 else []):
        say("symmetric ragged", M, N, K, g, dt, kern)
        Y = _run(X, dt, pd, g, kern, torch.float32)
        assert_close(out_to_f64(Y), ref, f"sym {M}x{N}x{K}")
    Xd = to_dev(X, bf16=(dt == "bf16"))
    a = awq.awq_linear_ex(Xd, *pd, group_size=g, out_dtype=torch.float32)
    b = awq.awq_linear_noalloc(Xd, *pd, group_size=g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --- fused projections (awq_linear_fused) -----------------------------------------------

@pytest.mark.parametrize("M,kernel", [(1, 0), (4, 0), (16, 1), (40, 0), (300, 0), (3, GEMM)])
@pytest.mark.parametrize("zp", [True, False])
def test_fused_qkv_parts(M, kernel, zp):
    """Q, K and V projections of one input (N = 4096, 1024 and 1000, the last
    ragged) in one call: each output against the fp64 oracle.  M <= 16 runs
    all three in one GEMV launch, larger M one GEMM per part."""
    torch = torch_mod()
    awq = _awq()
    K, g = 4096, 128
    Ns = (4096, 1024, 1000)
    X = wl.gen_activation(M, K, 190 + M, 191)
    packs = [_packed(wl.gen_weight(n, K, 192 + i), g, zero_point=zp) for i, n in enumerate(Ns)]
    say("fused qkv", M, kernel, zp)
    Ys = awq.awq_linear_fused(to_dev(X), [p[3] for p in packs], group_size=g,
                              out_dtype=torch.float32, kernel=kernel)
    torch.cuda.synchronize()
    for Y, (qw, sc, zr, _) in zip(Ys, packs):
        assert_close(out_to_f64(Y), linear64(X, qw, sc, zr, g), f"qkv M={M}")


@pytest.mark.parametrize("M,kernel,dt", [(1, 0, "f16"), (4, 0, "f16"), (4, 0, "bf16"), (16, GEMV, "f16"),
                                         (16, 0, "f16"), (24, 0, "bf16"), (64, 0, "f16"),
                                         (300, 0, "bf16"), (2, GEMM, "f16")])
def test_fused_gate_up_silu(M, kernel, dt):
    """The 7B-class MLP's gate and up projections (N = 11008, K = 4096) with
    the SiLU-mul epilogue: H = silu(X Wg^T) * (X Wu^T) against the fp64 oracle,
    fp32 and 16-bit output (the 16-bit output is the fp32 result rounded once).
    M = 16 and 24 with the automatic choice run each part on the batched-decode
    kernel, then the SiLU-mul kernel."""
    torch = torch_mod()
    awq = _awq()
    K, N, g = 4096, 11008, 128
    X = wl.gen_activation(M, K, 200 + M, 201, dt)
    gate = _packed(wl.gen_weight(N, K, 202), g)
    up = _packed(wl.gen_weight(N, K, 203), g)
    ref = gate_up_silu64(_x_f64(X, dt), gate[:3], up[:3], g)
    Xd = to_dev(X, bf16=(dt == "bf16"))
    say("fused gate/up silu", M, kernel, dt)
    H32 = awq.awq_linear_fused(Xd, [gate[3], up[3]], "silu_mul", g, torch.float32, kernel=kernel)
    H16 = awq.awq_linear_fused(Xd, [gate[3], up[3]], "silu_mul", g, kernel=kernel)
    torch.cuda.synchronize()
    got = out_to_f64(H32)
    assert torch.equal(H16, H32.to(H16.dtype))
    if M <= 32:
        # the GEMV, the batched-decode kernel and the 32-row tile multiply by
        # exact q - z
        rel, mx = assert_close(got, ref, f"gate/up M={M}")
        say("  rel_fro %.2e max_abs %.2e" % (rel, mx))
        return
    # Larger GEMM tiles round dequantized weights to fp16: each of gate and
    # up is then off by at most e = 2^-11 sum_k |x_k w_k| (their stated bound),
    # and H = silu(g) u by at most |silu'(g) u| e_g + |silu(g)| e_u (plus
    # second-order and fp32 terms).
    x64 = _x_f64(X, dt)
    dg = dequantize(unpack_codes(gate[0], K), gate[1], gate[2], g)
    du = dequantize(unpack_codes(up[0], K), up[1], up[2], g)
    yg, yu = x64 @ dg.T, x64 @ du.T
    eg = 2.0 ** -11 * (np.abs(x64) @ np.abs(dg).T)
    eu = 2.0 ** -11 * (np.abs(x64) @ np.abs(du).T)
    sig = 1.0 / (1.0 + np.exp(-yg))
    dsilu = sig * (1.0 + yg * (1.0 - sig))
    bound = np.abs(dsilu * yu) * eg + np.abs(yg * sig) * eu
    err = np.abs(got - ref)
    assert np.all(err <= 1.01 * bound + 1e-3 * eg * eu + 1e-5), float(np.max(err - bound))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= REL_FRO
    say("  rel_fro %.2e max_abs %.2e (bound holds)" % (rel, float(err.max())))


def test_fused_ragged_and_symmetric_pair():
    """A ragged gate/up pair (N = 200, g64, symmetric grid) through both paths."""
    torch = torch_mod()
    awq = _awq()
    K, N, g = 640, 200, 64
    gate = _packed(wl.gen_weight(N, K, 210), g, zero_point=False)
    up = _packed(wl.gen_weight(N, K, 211), g, zero_point=False)
    for M, kernel in ((3, 0), (3, GEMM), (50, 0)):
        X = wl.gen_activation(M, K, 212 + M, 213)
        say("fused ragged pair", M, kernel)
        H = awq.awq_linear_fused(to_dev(X), [gate[3], up[3]], "silu_mul", g, torch.float32,
                                 kernel=kernel)
        torch.cuda.synchronize()
        assert_close(out_to_f64(H), gate_up_silu64(X, gate[:3], up[:3], g), f"pair M={M}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fused_pair_partials_over_staged_rows(dt):
    """The GEMV's cross-wave partials reuse the start of LDS when they do not
    fit beside the staged data: the gate/up pair at M = 16, K = 2048 stages
    64 KiB of activation rows, and its partials (24 KiB) would take an
    8-wave workgroup past 80 KiB.  Ragged N, forced GEMV, against the fp64
    oracle."""
    torch = torch_mod()
    awq = _awq()
    M, K, N, g = 16, 2048, 1000, 128
    X = wl.gen_activation(M, K, 220, 221, dt)
    gate = _packed(wl.gen_weight(N, K, 222), g)
    up = _packed(wl.gen_weight(N, K, 223), g)
    say("fused pair, partials over staged rows", dt)
    H = awq.awq_linear_fused(to_dev(X, bf16=(dt == "bf16")), [gate[3], up[3]], "silu_mul", g,
                             torch.float32, kernel=GEMV)
    torch.cuda.synchronize()
    assert_close(out_to_f64(H), gate_up_silu64(_x_f64(X, dt), gate[:3], up[:3], g), f"pair {dt}")
