"""Pins for the oracle quantizer and packing (CPU only).

Each check is fixed by something other than the oracle's own formula: hand-
worked groups (tests/golden), the packed word of known codes, the error bound
of a uniform grid, a brute-force nearest-level search and exact equivariances.
"""

import json
import os

import numpy as np
import pytest

from oracle import (ORDER, QuantConfig, dequantize, pack_codes, quantize_groups,
                    quantize_pack, unpack_codes)

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "hand_worked_groups.json")))


def _group_array(values, g):
    row = np.zeros(g, dtype=np.float16)
    row[: len(values)] = np.array(values, dtype=np.float16)
    return row[None, :]


@pytest.mark.parametrize("grp", GOLD["groups"], ids=[g["name"] for g in GOLD["groups"]])
def test_hand_worked_group(grp):
    g = GOLD["group_size"]
    W = _group_array(grp["values"], g)
    q, sc, zr = quantize_groups(W, g)
    assert sc.shape == (1, 1) and zr.shape == (1, 1)
    assert int(sc.view(np.uint16)[0, 0]) == grp["scale_fp16_bits"]
    assert float(sc[0, 0]) == grp["scale"]
    assert int(zr[0, 0]) == grp["zero"]
    n = len(grp["codes"])
    assert q[0, :n].tolist() == grp["codes"]
    # the zero-filled tail maps to the zero point
    assert np.all(q[0, n:] == grp["zero"])
    if "dequant" in grp:
        deq = dequantize(q, sc, zr, g)
        assert deq[0, :n].tolist() == grp["dequant"]


def test_packed_word_of_known_codes():
    p = GOLD["packing"]
    q = np.array([p["codes"]], dtype=np.uint8)
    w = pack_codes(q)
    assert w.dtype == np.uint32 and w.shape == (1, 1)
    assert int(w[0, 0]) == p["word"]
    assert ORDER == (0, 2, 4, 6, 1, 3, 5, 7)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    assert np.array_equal(unpack_codes(pack_codes(q), 64), q)
    # each nibble moves independently: a single code lands in a single nibble
    for col in range(8):
        q1 = np.zeros((1, 8), dtype=np.uint8)
        q1[0, col] = 0xF
        assert int(pack_codes(q1)[0, 0]) == 0xF << (4 * ORDER.index(col))


def _random_w(N, K, seed, sigma=0.02):
    return (np.random.default_rng(seed).standard_normal((N, K)) * sigma).astype(np.float16)


@pytest.mark.parametrize("g", [64, 128])
def test_roundtrip_error_bound(g):
    W = _random_w(64, 512, 11)
    q, sc, zr = quantize_groups(W, g)
    assert q.max() <= 15 and zr.max() <= 15
    deq = dequantize(q, sc, zr, g)
    s_rep = np.repeat(sc.astype(np.float64), g, axis=1)
    err = np.abs(W.astype(np.float64) - deq)
    # every code: fp16 rounding of the scale can push the top level past 15
    assert np.all(err <= (0.5 + 15 * 2.0 ** -11) * s_rep)
    # codes below the top cannot have been clamped: half a step (+ fp32 rounding)
    below = q < 15
    assert np.all(err[below] <= 0.5 * s_rep[below] * (1 + 2.0 ** -20))
    # the zero point dequantizes to exactly zero
    zq = np.repeat(zr, g, axis=1)
    assert np.all(deq[q == zq] == 0.0)
    # every group uses its bottom code (the minimum maps to 0 or 0 lies in range)
    assert np.all(q.reshape(64, -1, g).min(axis=-1) == 0)


def test_brute_force_nearest_level():
    """For every unclamped weight the code is the nearest of the 16 levels,
    ties going to an even (q - z); near-ties decided by fp32 division may differ
    from the exact fp64 comparison only within a relative 2^-20."""
    g = 8
    W = _random_w(40, 64, 3, sigma=1.0)
    q, sc, zr = quantize_groups(W, g)
    v = W.astype(np.float64)
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            s = float(sc[n, k // g])
            z = int(zr[n, k // g])
            levels = (np.arange(16) - z) * s
            d = np.abs(v[n, k] - levels)
            best = np.flatnonzero(d == d.min())
            if len(best) == 2:          # exact tie: the even (q - z) wins
                best = [b for b in best if (b - z) % 2 == 0]
            if q[n, k] != best[0]:
                # allowed only at a near-tie (fp32 division vs exact)
                srt = np.sort(d)
                assert srt[1] - srt[0] <= 2.0 ** -20 * s * 16


def test_power_of_two_equivariance():
    W = _random_w(16, 256, 5)
    q, sc, zr = quantize_groups(W, 128)
    for e in (-3, 2):
        W2 = (W.astype(np.float32) * np.float32(2.0 ** e)).astype(np.float16)
        q2, sc2, zr2 = quantize_groups(W2, 128)
        assert np.array_equal(q2, q) and np.array_equal(zr2, zr)
        assert np.array_equal(sc2.astype(np.float64), sc.astype(np.float64) * 2.0 ** e)


def test_permutation_within_group():
    W = _random_w(4, 256, 9)
    perm = np.random.default_rng(1).permutation(128)
    Wp = W.copy()
    Wp[:, :128] = W[:, perm]
    q, sc, zr = quantize_groups(W, 128)
    qp, scp, zrp = quantize_groups(Wp, 128)
    assert np.array_equal(qp[:, :128], q[:, perm])
    assert np.array_equal(qp[:, 128:], q[:, 128:])
    assert np.array_equal(scp, sc) and np.array_equal(zrp, zr)


def test_lossless_grid_reproduces_codes():
    """Weights built exactly on a grid ((q - z) * 2^-6 with codes 0 and 15 present)
    quantize back to the same codes, zero and scale."""
    rng = np.random.default_rng(4)
    N, K, g = 6, 256, 128
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[:, ::g] = 0
    q[:, 1::g] = 15
    z = 5
    W = ((q.astype(np.float64) - z) * 2.0 ** -6).astype(np.float16)
    q2, sc, zr = quantize_groups(W, g)
    assert np.array_equal(q2, q)
    assert np.all(zr == z) and np.all(sc == np.float16(2.0 ** -6))


def test_scaled_quantization_multiplies_input_channels():
    """With s_k in {1, 1/2, 2} per input channel and W = grid / s, the values
    s*W lie exactly on a lossless grid, so the codes come back exactly.  Dividing
    by s, or applying s per output row, would not."""
    rng = np.random.default_rng(8)
    N, K, g = 5, 256, 128
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    q[:, ::g] = 0
    q[:, 1::g] = 15
    s = np.array([1.0, 0.5, 2.0, 1.0] * (K // 4), dtype=np.float32)
    grid = (q.astype(np.float64) - 7) * 2.0 ** -6
    W = (grid / s[None, :].astype(np.float64)).astype(np.float16)
    q2, sc, zr = quantize_groups(W, g, s)
    assert np.array_equal(q2, q)
    assert np.all(zr == 7) and np.all(sc == np.float16(2.0 ** -6))
    # unit s reproduces the unscaled quantizer bit for bit
    Wr = _random_w(8, 128, 2)
    a = quantize_groups(Wr, 128, np.ones(128, np.float32))
    b = quantize_groups(Wr, 128)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_config_validation():
    with pytest.raises(ValueError):
        QuantConfig(w_bit=3).check(128)
    with pytest.raises(ValueError):
        QuantConfig(group_size=128).check(192)
    QuantConfig(zero_point=False).check(128)
    qw, sc, zr = quantize_pack(_random_w(3, 256, 0), QuantConfig(group_size=64))
    assert qw.shape == (3, 32) and sc.shape == (3, 4) and zr.shape == (3, 4)
    qw, sc, zr = quantize_pack(_random_w(3, 256, 0), QuantConfig(group_size=64, zero_point=False))
    assert qw.shape == (3, 32) and sc.shape == (3, 4) and zr is None


# --- the symmetric grid (zero_point=False) --------------------------------------------

SYM = json.load(open(os.path.join(HERE, "golden", "hand_worked_symmetric.json")))


@pytest.mark.parametrize("grp", SYM["groups"], ids=[g["name"] for g in SYM["groups"]])
def test_symmetric_hand_worked_group(grp):
    g = SYM["group_size"]
    W = _group_array(grp["values"], g)
    q, sc, zr = quantize_groups(W, g, zero_point=False)
    assert zr is None and sc.shape == (1, 1)
    assert int(sc.view(np.uint16)[0, 0]) == grp["scale_fp16_bits"]
    assert float(sc[0, 0]) == grp["scale"]
    n = len(grp["codes"])
    assert q[0, :n].tolist() == grp["codes"]
    assert np.all(q[0, n:] == 8)
    if "dequant" in grp:
        assert dequantize(q, sc, None, g)[0, :n].tolist() == grp["dequant"]


@pytest.mark.parametrize("g", [64, 128])
def test_symmetric_roundtrip_bound_and_extremes(g):
    """Half a step for every weight (no level is ever clamped: |v|/s <= 7
    (1 + 2^-11) < 7.5), the largest magnitude of each group on level +-7, and
    code 0 (level -8) never used."""
    W = _random_w(64, 512, 12)
    q, sc, zr = quantize_groups(W, g, zero_point=False)
    deq = dequantize(q, sc, None, g)
    s_rep = np.repeat(sc.astype(np.float64), g, axis=1)
    v = W.astype(np.float64)
    assert np.all(np.abs(v - deq) <= 0.5 * s_rep * (1 + 2.0 ** -20))
    assert q.min() >= 1 and q.max() <= 15
    vg = np.abs(v).reshape(64, -1, g)
    arg = vg.argmax(axis=-1)
    qg = q.reshape(64, -1, g).astype(int) - 8
    ext = np.take_along_axis(qg, arg[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(ext) == 7)
    assert np.all(deq[q == 8] == 0.0)


def test_symmetric_brute_force_nearest_level():
    """Every code is the nearest of the 16 levels (c - 8) * s, ties going to
    an even q, except within fp32's rounding of the quotient at near-ties."""
    g = 8
    W = _random_w(40, 64, 13, sigma=1.0)
    q, sc, _ = quantize_groups(W, g, zero_point=False)
    v = W.astype(np.float64)
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            s = float(sc[n, k // g])
            levels = (np.arange(16) - 8) * s
            d = np.abs(v[n, k] - levels)
            best = np.flatnonzero(d == d.min())
            if len(best) == 2:
                best = [b for b in best if (b - 8) % 2 == 0]
            if q[n, k] != best[0]:
                srt = np.sort(d)
                assert srt[1] - srt[0] <= 2.0 ** -20 * s * 16


def test_symmetric_negation_and_scaling():
    """Negating W maps code c to 16 - c (q to -q) with the same steps; a power
    of two on W scales the steps exactly and keeps the codes.  A one-sided
    (asymmetric) or off-by-one grid breaks the first."""
    W = _random_w(16, 256, 14)
    q, sc, _ = quantize_groups(W, 128, zero_point=False)
    qn, scn, _ = quantize_groups(-W, 128, zero_point=False)
    assert np.array_equal(qn.astype(int), 16 - q.astype(int))
    assert np.array_equal(scn, sc)
    for e in (-3, 2):
        W2 = (W.astype(np.float32) * np.float32(2.0 ** e)).astype(np.float16)
        q2, sc2, _ = quantize_groups(W2, 128, zero_point=False)
        assert np.array_equal(q2, q)
        assert np.array_equal(sc2.astype(np.float64), sc.astype(np.float64) * 2.0 ** e)


def test_symmetric_scaled_input_channels():
    """With s on the input channels, v = fp32(s * W) is what gets quantized:
    a lossless symmetric grid divided by s comes back exactly."""
    rng = np.random.default_rng(15)
    N, K, g = 5, 256, 128
    q = rng.integers(1, 16, size=(N, K)).astype(np.uint8)
    q[:, ::g] = 1                      # -7: the largest magnitude of each group
    s = np.array([1.0, 0.5, 2.0, 1.0] * (K // 4), dtype=np.float32)
    grid = (q.astype(np.float64) - 8) * 2.0 ** -6
    W = (grid / s[None, :].astype(np.float64)).astype(np.float16)
    q2, sc, _ = quantize_groups(W, g, s, zero_point=False)
    assert np.array_equal(q2, q)
    assert np.all(sc == np.float16(2.0 ** -6))
