"""The seeded input generators: deterministic, the stated shapes and outlier counts."""

import numpy as np

import workloads as wl


def test_outlier_counts_match_one_percent():
    expect = {512: 5, 4096: 41, 5120: 51, 8192: 82, 11008: 110, 13824: 138, 28672: 287}
    for K, n in expect.items():
        assert wl.n_outliers(K) == n
        idx = wl.outlier_channels(K, 3)
        assert len(np.unique(idx)) == n and idx.max() < K


def test_generators_are_deterministic_and_chunk_invariant():
    a = wl.gen_weight(2100, 64, 5, row_seed=8)
    b = wl.gen_weight(2100, 64, 5, row_seed=8)
    assert np.array_equal(a, b)
    # rows come from one stream, so a prefix equals a smaller draw
    c = wl.gen_weight(700, 64, 5, row_seed=None)
    d = wl.gen_weight(2100, 64, 5, row_seed=None)
    assert np.array_equal(c, d[:700])
    x = wl.gen_activation(1500, 128, 1, 2)
    assert np.array_equal(x, wl.gen_activation(1500, 128, 1, 2))
    assert np.array_equal(wl.gen_activation(1, 128, 1, 2), x[:1])


def test_outlier_channels_are_scaled():
    K = 4096
    x = wl.gen_activation(256, K, 1, 2).astype(np.float64)
    idx = wl.outlier_channels(K, 2)
    rms = np.sqrt((x * x).mean(0))
    mask = np.zeros(K, bool)
    mask[idx] = True
    assert rms[mask].min() > 10 and rms[~mask].max() < 2


def test_bf16_bits_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    bits = wl.f32_to_bf16_bits(v)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_case_registry():
    cases = wl.all_cases()
    names = [c.name for c in cases]
    assert len(names) == len(set(names))
    assert sum(c.config == 4 for c in cases) == 4
    tiny = wl.tiny_cases()[0]
    assert (tiny.w_seed, tiny.x_seed, tiny.outlier_seed) == (0, 1, 2)
    gv = wl.gemv_cases()[0]
    assert gv.weight_bytes == 8_781_824
    assert wl.gemv_cases()[2].weight_bytes == 23_601_152
