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
