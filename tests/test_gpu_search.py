"""GPU parity: awq_scale_search against the oracle."""

import hashlib
import json
import os

import numpy as np
import pytest

import workloads as wl
from gpu_common import say, to_dev, to_np, torch_mod
from oracle import (DEFAULT_ALPHAS, QuantConfig, activation_mean_abs, quantize_pack,
                    scale_search, scale_vector)

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LOSS_RTOL = 1e-5


def _awq():
    import bit_weight_only_quantize_amd as awq
    return awq


def _gpu_search(X, W, g=128, alphas=None):
    res = _awq().awq_scale_search(to_dev(X), to_dev(W), group_size=g, alphas=alphas)
    torch_mod().cuda.synchronize()
    return res


def _check_against(res, ref, what):
    gap = np.sort(ref["losses"])[:2]
    say(what, "best", ref["best_index"], "runner-up gap", float((gap[1] - gap[0]) / gap[0]))
    rel = np.abs(res["losses"] - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, f"{what}: loss rel err {rel.max():.3e}"
    assert res["best_index"] == ref["best_index"]
    assert np.array_equal(to_np(res["s"]).view(np.uint32), ref["s"].view(np.uint32))
    assert np.array_equal(to_np(res["qweight"]), ref["qweight"])
    assert np.array_equal(to_np(res["scales"]).view(np.uint16), ref["scales"].view(np.uint16))
    assert np.array_equal(to_np(res["zeros"]), ref["zeros"])


@pytest.mark.parametrize("M,N,K,g", [(256, 192, 512, 128), (100, 77, 384, 64), (512, 256, 1024, 128)])
def test_small_search_matches_oracle(M, N, K, g):
    X = wl.gen_activation(M, K, 7 * M, 8 * M)
    W = wl.gen_weight(N, K, 9 * N)
    say("search small", M, N, K, g)
    res = _gpu_search(X, W, g)
    ref = scale_search(X, W, QuantConfig(group_size=g))
    _check_against(res, ref, f"search {M}x{N}x{K}")


def test_custom_alpha_grid():
    X = wl.gen_activation(128, 256, 3, 4)
    W = wl.gen_weight(64, 256, 5)
    alphas = [0.0, 0.25, 0.5, 0.75, 1.0]
    say("search custom alphas")
    res = _gpu_search(X, W, 128, alphas)
    ref = scale_search(X, W, QuantConfig(), np.array(alphas))
    _check_against(res, ref, "custom alphas")


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_full_search_layer_against_stored_oracle():
    """Search on one 4096x4096 layer with 4096 calibration tokens.  Expected
    values were written by tests/golden/make_search_golden.py, which calls only
    the oracle."""
    gold = json.load(open(os.path.join(HERE, "golden", "search_4096.json")))
    case = wl.search_case()
    X = case.activation()
    W = case.weight()
    say("search full 4096^3")
    res = _gpu_search(X, W)
    losses = np.array(gold["losses"], dtype=np.float64)
    rel = np.abs(res["losses"] - losses) / losses
    assert rel.max() <= LOSS_RTOL, f"loss rel err {rel.max():.3e}"
    assert res["best_index"] == gold["best_index"]
    assert _sha(to_np(res["s"]).view(np.uint32)) == gold["sha256_s"]
    assert _sha(to_np(res["qweight"])) == gold["sha256_qweight"]
    assert _sha(to_np(res["scales"]).view(np.uint16)) == gold["sha256_scales"]
    assert _sha(to_np(res["zeros"])) == gold["sha256_zeros"]
    # the whole s-table: every candidate's s vector is bit-identical to the oracle's
    xbar = activation_mean_abs(X)
    s_best = scale_vector(xbar, DEFAULT_ALPHAS[gold["best_index"]])
    assert np.array_equal(to_np(res["s"]), s_best)
