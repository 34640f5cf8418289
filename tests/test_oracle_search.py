"""Pins for the oracle activation statistic, scaling and alpha search (CPU only)."""

import numpy as np
import pytest

from oracle import (DEFAULT_ALPHAS, QuantConfig, activation_mean_abs, dequantize,
                    quantize_groups, quantize_pack, reference_output, scale_search,
                    scale_table, scale_vector, scaled_activation, search_loss)
from workloads import gen_activation, gen_weight


def test_mean_abs_closed_form():
    X = np.array([[1.0, -2.0, 0.5], [-3.0, 2.0, 0.5]], dtype=np.float16)
    assert activation_mean_abs(X).tolist() == [2.0, 2.0, 0.5]


def test_mean_abs_is_order_independent():
    X = gen_activation(64, 256, 1, 2)
    a = activation_mean_abs(X)
    b = activation_mean_abs(X[::-1])
    c = np.abs(X.astype(np.float64))[np.random.default_rng(0).permutation(64)].sum(0) / 64
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_mean_abs_exact_beyond_fp64_summation():
    """Column sums of ~34000 rows near fp16's maximum exceed 2^53 units of
    2^-24, where fp64 accumulation stops being exact; a few subnormal
    magnitudes mixed in make plain fp64 summation round differently.  The
    statistic must still be the exact mean rounded once (compared with exact
    rational arithmetic), and the naive fp64 sum must miss it on some column
    (so this pin separates the two)."""
    from fractions import Fraction
    M, K = 34278, 8
    rng = np.random.default_rng(0)
    X = np.full((M, K), 65504.0)
    for k in range(K):
        X[rng.integers(0, M, size=int(rng.integers(1, 40))), k] = rng.integers(1, 1024) * 2.0 ** -24
        X[rng.integers(0, M, size=3), k] = 65504.0 - 32 * rng.integers(1, 60)
    X[::7, 2] *= -1.0                        # magnitudes, not values
    X = X.astype(np.float16)
    got = activation_mean_abs(X)
    naive = np.abs(X.astype(np.float64)).sum(axis=0) / np.float64(M)
    for k in range(K):
        exact = sum((Fraction(abs(float(v))) for v in X[:, k]), Fraction(0)) / M
        assert got[k] == float(exact), k
    assert np.any(naive != got)


def test_two_channel_scale_closed_form():
    xbar = np.array([1.0, 4.0])
    # alpha = 1/2: t = (1, 2), sqrt(max*min) = sqrt(2): s = (2^-1/2, 2^1/2)
    s = scale_vector(xbar, 0.5)
    assert s.dtype == np.float32
    assert s.tolist() == [np.float32(2 ** -0.5), np.float32(2 ** 0.5)]
    # alpha = 0: plain rounding, s = 1 exactly
    assert scale_vector(xbar, 0.0).tolist() == [1.0, 1.0]
    # alpha = 1: t = xbar, s = xbar / 2
    assert scale_vector(xbar, 1.0).tolist() == [0.5, 2.0]


def test_scale_table_properties():
    X = gen_activation(128, 512, 11, 12)
    xbar = activation_mean_abs(X)
    tab = scale_table(xbar)
    assert tab.shape == (20, 512) and tab.dtype == np.float32
    assert np.all(tab[0] == 1.0)
    assert np.all(tab > 0)
    # larger statistic -> larger scale, for every alpha > 0 (salient channels
    # receive the larger factors)
    order = np.argsort(xbar, kind="stable")
    for j in range(1, 20):
        assert np.all(np.diff(tab[j][order].astype(np.float64)) >= 0)
    # geometric centring: max*min is 1 up to the fp32 rounding
    for j in range(20):
        assert abs(float(tab[j].max()) * float(tab[j].min()) - 1.0) < 1e-6
    assert np.allclose(DEFAULT_ALPHAS, np.arange(20) / 20, rtol=0, atol=0)


def test_prequantization_equivalence():
    """(X/s)(sW)^T = XW^T in exact arithmetic: fp64 agreement to 1e-13 for every alpha."""
    X = gen_activation(16, 256, 21, 22)
    W = gen_weight(12, 256, 23)
    xbar = activation_mean_abs(X)
    X64, W64 = X.astype(np.float64), W.astype(np.float64)
    ref = X64 @ W64.T
    for a in DEFAULT_ALPHAS:
        s = scale_vector(xbar, a).astype(np.float64)
        lhs = (X64 / s[None, :]) @ (W64 * s[None, :]).T
        assert np.max(np.abs(lhs - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_scaled_activation_folds_the_inverse_scale():
    """A = fp16(X/s) is within fp16 rounding of X/s (a scale applied on the wrong
    axis or multiplied instead of divided would be off by O(1))."""
    X = gen_activation(8, 256, 31, 32)
    s = scale_vector(activation_mean_abs(X), 0.7)
    A = scaled_activation(X, s).astype(np.float64)
    exact = X.astype(np.float64) / s.astype(np.float64)[None, :]
    assert np.all(np.abs(A - exact) <= 2.0 ** -11 * np.abs(exact) + 2.0 ** -24)
    assert np.array_equal(scaled_activation(X, np.ones(256, np.float32)), X)


def _lossless(N, K, g, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[:, ::g] = 0
    q[:, 1::g] = 15
    return ((q.astype(np.float64) - 6) * 2.0 ** -7).astype(np.float16)


def test_loss_zero_on_lossless_grid():
    W = _lossless(10, 256, 128, 1)
    X = gen_activation(12, 256, 41, 42)
    L, _ = search_loss(X, W, np.ones(256, np.float32))
    assert L == 0.0


def test_loss_invariances():
    X = gen_activation(16, 256, 51, 52)
    W = gen_weight(20, 256, 53)
    s = scale_vector(activation_mean_abs(X), 0.5)
    L, codes = search_loss(X, W, s)
    # s -> s/2: A doubles, sW halves, both exactly: L is bit-identical
    L2, codes2 = search_loss(X, W, (s / np.float32(2)).astype(np.float32))
    assert L2 == L
    assert np.array_equal(codes2[0], codes[0]) and np.array_equal(codes2[2], codes[2])
    # X -> 2X: every error doubles exactly: L x 4
    L4, _ = search_loss((X.astype(np.float32) * 2).astype(np.float16), W, s)
    assert L4 == 4 * L


def test_loss_matches_python_loops():
    M, N, K, g = 3, 4, 16, 8
    X = gen_activation(M, K, 61, 62)
    W = gen_weight(N, K, 63)
    s = scale_vector(activation_mean_abs(X), 0.35)
    L, (q, sc, zr) = search_loss(X, W, s, QuantConfig(group_size=g))
    A = scaled_activation(X, s)
    tot = 0.0
    for m in range(M):
        for n in range(N):
            yr = sum(float(X[m, k]) * float(W[n, k]) for k in range(K))
            yq = sum(float(A[m, k]) * (float(q[n, k]) - float(zr[n, k // g])) * float(sc[n, k // g])
                     for k in range(K))
            tot += (yr - yq) ** 2
    assert abs(L - tot) <= 1e-12 * tot


def test_alpha_zero_is_plain_rounding():
    X = gen_activation(32, 256, 71, 72)
    W = gen_weight(16, 256, 73)
    res = scale_search(X, W)
    s0 = scale_vector(activation_mean_abs(X), 0.0)
    assert np.all(s0 == 1.0)
    L0, (q0, sc0, zr0) = search_loss(X, W, s0)
    q_plain, sc_plain, zr_plain = quantize_groups(W, 128)
    assert np.array_equal(q0, q_plain) and np.array_equal(sc0, sc_plain) and np.array_equal(zr0, zr_plain)
    assert res["losses"][0] == L0
    # the search can only improve on plain rounding
    assert res["losses"][res["best_index"]] <= L0
    assert res["best_index"] == int(np.argmin(res["losses"]))


def test_search_returns_consistent_artifacts():
    X = gen_activation(64, 512, 81, 82)
    W = gen_weight(32, 512, 83)
    res = scale_search(X, W)
    j = res["best_index"]
    s = scale_vector(activation_mean_abs(X), DEFAULT_ALPHAS[j])
    assert np.array_equal(res["s"], s)
    qw, sc, zr = quantize_pack(W, QuantConfig(), s)
    assert np.array_equal(res["qweight"], qw)
    assert np.array_equal(res["scales"], sc) and np.array_equal(res["zeros"], zr)
    # on outlier activations the activation-aware scaling beats plain rounding
    assert res["losses"][j] < res["losses"][0]


def test_reference_output_blocked():
    X = gen_activation(5, 128, 91, 92)
    W = gen_weight(70, 128, 93)
    assert np.array_equal(reference_output(X, W, block=16),
                          X.astype(np.float64) @ W.astype(np.float64).T)


@pytest.mark.parametrize("grid,want", [([0.35, 0.35], 0), ([0.9, 0.35, 0.35], 1),
                                       ([0.35, 0.9, 0.35], 0), ([0.9, 0.9, 0.35, 0.35], 2)])
def test_tie_break_takes_the_first_minimum(grid, want):
    """Reading R16: the smallest index attaining the minimum.  A repeated alpha
    gives bit-identical losses (the loss is a deterministic function of alpha),
    so a rule that kept the last minimum would return the later copy.  The
    data give L(0.35) < L(0.9) (checked), so 0.35's first copy must win."""
    X = gen_activation(256, 512, 150, 151)
    W = gen_weight(192, 512, 152)
    res = scale_search(X, W, QuantConfig(), np.array(grid))
    L = res["losses"]
    xbar = activation_mean_abs(X)
    l35 = search_loss(X, W, scale_vector(xbar, 0.35))[0]
    l90 = search_loss(X, W, scale_vector(xbar, 0.9))[0]
    assert l35 < l90
    for i, a in enumerate(grid):
        assert L[i] == (l35 if a == 0.35 else l90)
    assert res["best_index"] == want


def test_symmetric_search_alpha_zero_is_plain_symmetric_rounding():
    """zero_point=False runs the same search over the symmetric grid: alpha 0
    reproduces the plain symmetric quantizer, the packed result carries no
    zero points, and the loss matches a direct evaluation."""
    X = gen_activation(32, 256, 171, 172)
    W = gen_weight(16, 256, 173)
    cfg = QuantConfig(zero_point=False)
    res = scale_search(X, W, cfg)
    assert res["zeros"] is None
    L0, (q0, sc0, zr0) = search_loss(X, W, np.ones(256, np.float32), cfg)
    q_plain, sc_plain, _ = quantize_groups(W, 128, zero_point=False)
    assert zr0 is None and np.array_equal(q0, q_plain) and np.array_equal(sc0, sc_plain)
    assert res["losses"][0] == L0
    qw, sc, zr = quantize_pack(W, cfg, res["s"])
    assert np.array_equal(res["qweight"], qw) and zr is None


# --- duo scaling -----------------------------------------------------------------------

def test_duo_scaling_closed_forms():
    from oracle import weight_mean_abs
    W = np.array([[1.0, -4.0], [-3.0, 2.0]], dtype=np.float16)
    assert weight_mean_abs(W).tolist() == [2.0, 3.0]
    # xbar = (1, 4), wbar = (4, 1), alpha = 1/2: t = (1/2, 2), sqrt(max*min) = 1
    s = scale_vector(np.array([1.0, 4.0]), 0.5, np.array([4.0, 1.0]))
    assert s.tolist() == [0.5, 2.0]
    # alpha = 1 ignores the weights exactly (wbar^0 = 1)
    X = gen_activation(64, 256, 301, 302)
    Wr = gen_weight(32, 256, 303)
    xbar, wbar = activation_mean_abs(X), weight_mean_abs(Wr)
    assert np.array_equal(scale_vector(xbar, 1.0, wbar), scale_vector(xbar, 1.0))
    # alpha = 0 equalizes the weight magnitudes: s_k * wbar_k is one constant
    s0 = scale_vector(xbar, 0.0, wbar).astype(np.float64)
    prod = s0 * wbar
    assert np.max(np.abs(prod / prod[0] - 1.0)) < 2.0 ** -22
    # a factor 4 on every weight magnitude scales t by 4^-(1/2) = 1/2 at alpha
    # 1/2, which the normalization removes exactly
    assert np.array_equal(scale_vector(xbar, 0.5, 4.0 * wbar), scale_vector(xbar, 0.5, wbar))


def test_duo_search_uses_both_statistics():
    """The duo search's candidate j equals scale_vector(xbar, alpha_j, wbar);
    its alpha-1 candidate coincides with the plain search's."""
    from oracle import weight_mean_abs
    X = gen_activation(64, 256, 311, 312)
    W = gen_weight(24, 256, 313)
    duo = scale_search(X, W, duo_scaling=True)
    plain = scale_search(X, W, alphas=np.array([1.0]))
    one = scale_search(X, W, alphas=np.array([1.0]), duo_scaling=True)
    assert one["losses"][0] == plain["losses"][0]
    s = scale_vector(activation_mean_abs(X), DEFAULT_ALPHAS[duo["best_index"]], weight_mean_abs(W))
    assert np.array_equal(duo["s"], s)


# --- weight clipping ------------------------------------------------------------------

@pytest.mark.parametrize("zp", [True, False])
def test_clip_factor_one_is_plain_quantization(zp):
    from oracle import clip_search, quantize_group_clipped
    W = gen_weight(16, 256, 321)
    v = W.astype(np.float32).reshape(16, 2, 128)
    q, s_h, z = quantize_group_clipped(v, np.float32(1.0), 128, zp)
    qr, sr, zr = quantize_groups(W, 128, zero_point=zp)
    assert np.array_equal(q.reshape(16, 256).astype(np.uint8), qr) and np.array_equal(s_h, sr)
    X = gen_activation(32, 256, 322, 323)
    ones = np.ones(256, np.float32)
    r = clip_search(X, W, ones, QuantConfig(zero_point=zp), grid=np.array([1.0], np.float32))
    assert np.all(r["clip_index"] == 0) and np.array_equal(r["q"], qr)


@pytest.mark.parametrize("zp", [True, False])
def test_clip_choice_against_direct_output_error(zp):
    """The chosen factor minimizes ||A_g (v - deq_c(v))||^2 computed directly
    by loops over tokens (not through the Gram matrix), and the errors agree."""
    from oracle import CLIP_GRID, clip_search, quantize_group_clipped
    M, N, K, g = 24, 6, 128, 64
    X = gen_activation(M, K, 331, 332)
    W = gen_weight(N, K, 333)
    s = scale_vector(activation_mean_abs(X), 0.5)
    r = clip_search(X, W, s, QuantConfig(group_size=g, zero_point=zp))
    A = scaled_activation(X, s).astype(np.float64)
    v = (s[None, :] * W.astype(np.float32)).reshape(N, K // g, g)
    for n in range(N):
        for gi in range(K // g):
            errs = []
            for c in CLIP_GRID:
                q, s_h, z = quantize_group_clipped(v[n:n + 1, gi:gi + 1], c, g, zp)
                d = v[n, gi].astype(np.float64) - (q[0, 0].astype(np.float64) - float(z[0, 0])) * float(s_h[0, 0])
                e = 0.0
                for m in range(M):
                    t = sum(float(A[m, gi * g + k]) * float(d[k]) for k in range(g))
                    e += t * t
                errs.append(e)
            errs = np.array(errs)
            i = int(r["clip_index"][n, gi])
            assert abs(r["errors"][n, gi] - errs[i]) <= 1e-9 * errs[i] + 1e-300
            assert errs[i] <= errs.min() * (1 + 1e-12)
            assert i == int(np.flatnonzero(errs <= errs.min() * (1 + 1e-12))[0])


def test_clip_prefers_shrinking_an_unused_outlier():
    """A group whose largest weight meets an input channel that is always zero:
    shrinking the range costs nothing there and refines every other weight, so
    a factor below 1 wins, and with all activations zero every error is 0 and
    the first factor (1) wins."""
    from oracle import clip_search
    rng = np.random.default_rng(341)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float16)
    W[:, 5] = np.float16(0.5)
    X = rng.standard_normal((64, 128)).astype(np.float16)
    X[:, 5] = 0
    ones = np.ones(128, np.float32)
    r = clip_search(X, W, ones, QuantConfig())
    assert np.all(r["clip_index"] > 0)
    r0 = clip_search(np.zeros((8, 128), np.float16), W, ones, QuantConfig())
    assert np.all(r0["clip_index"] == 0) and np.all(r0["errors"] == 0)


def test_search_with_clip_packs_the_clipped_codes():
    from oracle import clip_search, pack_codes
    X = gen_activation(64, 256, 351, 352)
    W = gen_weight(16, 256, 353)
    r = scale_search(X, W, apply_clip=True)
    c = clip_search(X, W, r["s"], QuantConfig())
    assert np.array_equal(r["qweight"], pack_codes(c["q"])) and np.array_equal(r["clip_index"], c["clip_index"])
    plain = scale_search(X, W)
    assert np.array_equal(r["losses"], plain["losses"]) and r["best_index"] == plain["best_index"]
