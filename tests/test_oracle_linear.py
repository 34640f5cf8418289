"""Pins for the oracle dequant-matmul (CPU only)."""

import numpy as np
import pytest

from oracle import (dequantize, linear64, linear_naive, pack_codes, quantize_groups,
                    quantize_pack, QuantConfig)


def _w(N, K, seed):
    return (np.random.default_rng(seed).standard_normal((N, K)) * 0.02).astype(np.float16)


def test_one_hot_rows_select_dequantized_columns():
    """X = identity: Y[k][n] must equal deq[n][k] exactly (catches a transposed
    operand or a wrong group index)."""
    N, K, g = 24, 256, 64
    W = _w(N, K, 1)
    q, sc, zr = quantize_groups(W, g)
    qw = pack_codes(q)
    X = np.eye(K, dtype=np.float16)
    Y = linear64(X, qw, sc, zr, g)
    assert np.array_equal(Y, dequantize(q, sc, zr, g).T)


def test_naive_loop_agrees():
    M, N, K, g = 3, 5, 256, 128
    W = _w(N, K, 2)
    X = np.random.default_rng(3).standard_normal((M, K)).astype(np.float16)
    q, sc, zr = quantize_groups(W, g)
    Y = linear64(X, pack_codes(q), sc, zr, g)
    Yn = linear_naive(X, q, sc, zr, g)
    assert np.max(np.abs(Y - Yn)) <= 1e-12 * np.max(np.abs(Yn))


def test_lossless_grid_gives_exact_xwt():
    rng = np.random.default_rng(5)
    M, N, K, g = 4, 7, 256, 128
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[:, ::g] = 0
    q[:, 1::g] = 15
    W = ((q.astype(np.float64) - 3) * 2.0 ** -5).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    qw, sc, zr = quantize_pack(W, QuantConfig(group_size=g))
    Y = linear64(X, qw, sc, zr, g)
    assert np.array_equal(Y, X.astype(np.float64) @ W.astype(np.float64).T)


def test_sampled_rows_and_cols_match_full():
    M, N, K, g = 6, 40, 256, 128
    W = _w(N, K, 6)
    X = np.random.default_rng(7).standard_normal((M, K)).astype(np.float16)
    qw, sc, zr = quantize_pack(W, QuantConfig(group_size=g))
    full = linear64(X, qw, sc, zr, g)
    rows = np.array([0, 5, 2])
    cols = np.array([39, 0, 17, 17])
    part = linear64(X, qw, sc, zr, g, rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


@pytest.mark.parametrize("g", [64, 128])
def test_error_vs_unquantized_is_small(g):
    """The quantized layer approximates X*W^T: relative Frobenius error of a
    16-level grid on Gaussian weights is a few percent, far from 1."""
    M, N, K = 8, 64, 512
    W = _w(N, K, 8)
    X = np.random.default_rng(9).standard_normal((M, K)).astype(np.float16)
    qw, sc, zr = quantize_pack(W, QuantConfig(group_size=g))
    Y = linear64(X, qw, sc, zr, g)
    Yr = X.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(Y - Yr) / np.linalg.norm(Yr)
    assert 0.01 < rel < 0.2


def test_symmetric_grid_matches_python_loops():
    """Without zero points (zeros=None: every zero is 8) the fp64 product
    equals a pure-Python loop over (code - 8) * scale."""
    W = _w(12, 256, 77)
    X = (np.random.default_rng(78).standard_normal((3, 256))).astype(np.float16)
    q, sc, zr = quantize_groups(W, 64, zero_point=False)
    assert zr is None
    got = linear64(X, pack_codes(q), sc, None, 64)
    ref = linear_naive(X, q, sc, None, 64)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_silu_identities():
    """silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1), silu(0) = 0, the
    large-|x| limits, and agreement with x * scipy's logistic function."""
    from scipy.special import expit
    from oracle import silu64
    x = np.linspace(-30, 30, 6001)
    assert np.allclose(silu64(x) - silu64(-x), x, rtol=1e-14, atol=1e-14)
    assert silu64(0.0) == 0.0
    assert abs(silu64(40.0) - 40.0) < 1e-15 and abs(silu64(-40.0)) < 1e-15
    assert np.allclose(silu64(x), x * expit(x), rtol=1e-15, atol=1e-300)


def test_gate_up_silu_matches_loops():
    """The fused gate/up oracle equals silu applied to a pure-Python loop's
    gate product, times the loop's up product."""
    from oracle import gate_up_silu64, silu64
    Wg, Wu = _w(6, 128, 91), _w(6, 128, 92)
    X = (np.random.default_rng(93).standard_normal((2, 128))).astype(np.float16)
    gq, gs, gz = quantize_groups(Wg, 64)
    uq, us, uz = quantize_groups(Wu, 64)
    got = gate_up_silu64(X, (pack_codes(gq), gs, gz), (pack_codes(uq), us, uz), 64)
    yg = linear_naive(X, gq, gs, gz, 64)
    yu = linear_naive(X, uq, us, uz, 64)
    ref = np.array([[float(a) / (1.0 + np.exp(-float(a))) * float(b) for a, b in zip(ra, rb)]
                    for ra, rb in zip(yg, yu)])
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
