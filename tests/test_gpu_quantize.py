"""GPU parity: awq_quantize_pack against the oracle, bit for bit."""

import json
import os

import numpy as np
import pytest

import workloads as wl
from gpu_common import dev, say, to_dev, to_np, torch_mod
from oracle import QuantConfig, pack_codes, quantize_groups, quantize_pack

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _awq():
    import bit_weight_only_quantize_amd as awq
    return awq


def _gpu_pack(W, g, s=None, zero_point=True):
    awq = _awq()
    qw, sc, zr = awq.awq_quantize_pack(to_dev(W), group_size=g,
                                       s=None if s is None else to_dev(s), zero_point=zero_point)
    torch_mod().cuda.synchronize()
    return to_np(qw), to_np(sc), None if zr is None else to_np(zr)


def _assert_same(gpu, ref, what):
    names = ("qweight", "scales", "zeros")
    for a, b, nm in zip(gpu, ref, names):
        if a is None or b is None:
            assert a is None and b is None, (what, nm)
            continue
        a = np.asarray(a)
        b = np.asarray(b)
        if nm == "scales":
            a, b = a.view(np.uint16), b.view(np.uint16)
        assert a.shape == b.shape, (what, nm, a.shape, b.shape)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{what}: {nm} differs at {len(bad)} places, first {bad[:3].tolist()}"


def test_hand_worked_groups_on_gpu():
    gold = json.load(open(os.path.join(HERE, "golden", "hand_worked_groups.json")))
    g = gold["group_size"]
    rows = []
    for grp in gold["groups"]:
        r = np.zeros(g, dtype=np.float16)
        r[: len(grp["values"])] = np.array(grp["values"], dtype=np.float16)
        rows.append(r)
    W = np.stack(rows)
    say("hand-worked groups", W.shape)
    qw, sc, zr = _gpu_pack(W, g)
    from oracle import unpack_codes
    q = unpack_codes(qw, g)
    for i, grp in enumerate(gold["groups"]):
        n = len(grp["codes"])
        assert q[i, :n].tolist() == grp["codes"], grp["name"]
        assert int(sc.view(np.uint16)[i, 0]) == grp["scale_fp16_bits"], grp["name"]
        assert int(zr[i, 0]) == grp["zero"], grp["name"]
    # packed word of codes 0..7: the layout constant
    Wp = ((np.arange(8, dtype=np.float64) - 0) * 2.0 ** -6).astype(np.float16)
    Wrow = np.zeros((1, 128), np.float16)
    Wrow[0, :8] = Wp
    Wrow[0, 8] = np.float16(15 * 2.0 ** -6)     # pins the range to [0, 15 * 2^-6]
    qw1, _, _ = _gpu_pack(Wrow, 128)
    assert int(qw1[0, 0]) == gold["packing"]["word"]


SMALL = [(77, 192, 64), (16, 512, 128), (300, 1024, 64), (5, 128, 128)]


@pytest.mark.parametrize("N,K,g", SMALL)
def test_ragged_and_small(N, K, g):
    W = wl.gen_weight(N, K, 1000 + N, row_seed=7)
    say("quantize ragged", N, K, g)
    _assert_same(_gpu_pack(W, g), quantize_pack(W, QuantConfig(group_size=g)), f"{N}x{K}g{g}")
    s = np.exp(np.random.default_rng(N).standard_normal(K)).astype(np.float32)
    _assert_same(_gpu_pack(W, g, s), quantize_pack(W, QuantConfig(group_size=g), s),
                 f"{N}x{K}g{g} scaled")


def test_degenerate_rows():
    K = 256
    W = np.zeros((4, K), np.float16)
    W[1] = np.float16(0.5)                            # constant positive rows
    W[2, :128] = -np.float16(3.0)
    W[3] = np.linspace(-1e-7, 1e-7, K).astype(np.float16)   # subnormal fp16 weights
    say("quantize degenerate")
    _assert_same(_gpu_pack(W, 128), quantize_pack(W, QuantConfig()), "degenerate")


FULL = [(c.N, c.K, c.group_size, c.row_seed, c.w_seed)
        for c in wl.tiny_cases()[:1] + wl.gemv_cases(Ms=(1,))]
FULL += [(13824, 5120, 64, None, 300), (5120, 13824, 128, None, 310), (4096, 4096, 128, None, 500)]


@pytest.mark.parametrize("N,K,g,row_seed,seed", FULL)
def test_full_layers_bit_exact(N, K, g, row_seed, seed):
    W = wl.gen_weight(N, K, seed, row_seed)
    say("quantize full", N, K, g)
    _assert_same(_gpu_pack(W, g), quantize_pack(W, QuantConfig(group_size=g)), f"{N}x{K}g{g}")


@pytest.mark.parametrize("case", wl.prefill_cases(dtypes=("f16",)), ids=lambda c: c.name)
def test_prefill_layers_sampled_rows(case):
    """70B-class layers: the GPU packs the whole matrix; the oracle checks 512
    sampled rows (quantization is row-independent) plus the first and last."""
    W = case.weight()
    say("quantize prefill", case.N, case.K)
    qw, sc, zr = _gpu_pack(W, case.group_size)
    rows = np.unique(np.concatenate([[0, case.N - 1],
                                     np.random.default_rng(5).choice(case.N, 512, replace=False)]))
    ref = quantize_pack(W[rows], QuantConfig(group_size=case.group_size))
    _assert_same((qw[rows], sc[rows], zr[rows]), ref, case.name)


def test_with_activation_scale_vector():
    case = wl.search_case()
    W = case.weight()
    X = case.activation(M=512)
    from oracle import activation_mean_abs, scale_vector
    s = scale_vector(activation_mean_abs(X), 0.5)
    say("quantize scaled 4096x4096")
    _assert_same(_gpu_pack(W, 128, s), quantize_pack(W, QuantConfig(), s), "scaled")


def test_nonfinite_count():
    awq = _awq()
    torch = torch_mod()
    W = wl.gen_weight(8, 256, 3)
    W[2, 5] = np.float16(np.nan)
    W[7, 200] = np.float16(np.inf)
    W[0, 0] = -np.float16(np.inf)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    say("quantize nonfinite")
    awq.awq_quantize_pack(to_dev(W), 128, nonfinite_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 3
    # rows without non-finite values are unaffected
    qw, sc, zr = _gpu_pack(W, 128)
    ref = quantize_pack(W[[1, 3, 4, 5, 6]], QuantConfig())
    _assert_same((qw[[1, 3, 4, 5, 6]], sc[[1, 3, 4, 5, 6]], zr[[1, 3, 4, 5, 6]]), ref, "finite rows")


def test_empty_is_noop():
    awq = _awq()
    torch = torch_mod()
    W = torch.empty((0, 256), dtype=torch.float16, device=dev())
    qw, sc, zr = awq.awq_quantize_pack(W, 128)
    assert qw.shape == (0, 32)


# --- the symmetric grid (zero_point=False) ----------------------------------------------

def test_symmetric_hand_worked_groups_on_gpu():
    gold = json.load(open(os.path.join(HERE, "golden", "hand_worked_symmetric.json")))
    g = gold["group_size"]
    W = np.zeros((len(gold["groups"]), g), dtype=np.float16)
    for i, grp in enumerate(gold["groups"]):
        W[i, : len(grp["values"])] = np.array(grp["values"], dtype=np.float16)
    say("symmetric hand-worked groups", W.shape)
    qw, sc, zr = _gpu_pack(W, g, zero_point=False)
    assert zr is None
    from oracle import unpack_codes
    q = unpack_codes(qw, g)
    for i, grp in enumerate(gold["groups"]):
        n = len(grp["codes"])
        assert q[i, :n].tolist() == grp["codes"], grp["name"]
        assert np.all(q[i, n:] == 8), grp["name"]
        assert int(sc.view(np.uint16)[i, 0]) == grp["scale_fp16_bits"], grp["name"]


@pytest.mark.parametrize("N,K,g", SMALL)
def test_symmetric_ragged_and_small(N, K, g):
    W = wl.gen_weight(N, K, 1100 + N, row_seed=8)
    cfg = QuantConfig(group_size=g, zero_point=False)
    say("symmetric quantize ragged", N, K, g)
    _assert_same(_gpu_pack(W, g, zero_point=False), quantize_pack(W, cfg), f"sym {N}x{K}g{g}")
    s = np.exp(np.random.default_rng(N + 1).standard_normal(K)).astype(np.float32)
    _assert_same(_gpu_pack(W, g, s, zero_point=False), quantize_pack(W, cfg, s),
                 f"sym {N}x{K}g{g} scaled")


@pytest.mark.parametrize("case", wl.gemv_cases(Ms=(1,)), ids=lambda c: c.name)
def test_symmetric_decode_layers(case):
    """The 7B-class layers quantized without zero points, every word, scale
    and code bit-identical to the oracle's."""
    W = case.weight()
    say("symmetric quantize layer", case.name)
    _assert_same(_gpu_pack(W, 128, zero_point=False),
                 quantize_pack(W, QuantConfig(zero_point=False)), case.name)


# --- dequantize (the pseudo-quantized weights) --------------------------------------------

@pytest.mark.parametrize("N,K,g,zp", [(77, 192, 64, True), (300, 1024, 128, False),
                                      (4096, 4096, 128, True), (11008, 4096, 128, False)])
def test_dequantize_bit_exact(N, K, g, zp):
    """awq_dequantize of packed weights: fp32 output equals the oracle's exact
    (q - z) * s; fp16 output equals it rounded once to fp16 (nearest even)."""
    from oracle import dequantize, unpack_codes
    awq = _awq()
    torch = torch_mod()
    W = wl.gen_weight(N, K, 1200 + N, row_seed=9)
    qw, sc, zr = quantize_pack(W, QuantConfig(group_size=g, zero_point=zp))
    ref = dequantize(unpack_codes(qw, K), sc, zr, g)
    pd = (to_dev(qw), to_dev(sc), None if zr is None else to_dev(zr))
    say("dequantize", N, K, g, zp)
    o32 = awq.awq_dequantize(*pd, K, group_size=g)
    o16 = awq.awq_dequantize(*pd, K, group_size=g, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(o32.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(to_np(o16).view(np.uint16), ref.astype(np.float16).view(np.uint16))
