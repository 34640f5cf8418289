"""GPU check of awq_linear_noalloc (static device scratch, no allocation)
through the C ABI: two calls in a row, the second smaller, each bit-identical
to awq_linear_ws on the same inputs with a workspace of its own."""

import ctypes

import numpy as np
import pytest

import workloads as wl
from gpu_common import assert_close, dev, say, to_dev, torch_mod
from oracle import QuantConfig, bf16_bits_to_f32, linear64, quantize_pack

pytestmark = pytest.mark.gpu


def _call_noalloc(awq, Xd, pd, M, N, K, g, out):
    torch = torch_mod()
    qw, sc, zr = pd
    st = awq.lib.awq_linear_noalloc(
        ctypes.c_void_p(Xd.data_ptr()), 0 if Xd.dtype == torch.float16 else 1,
        ctypes.c_void_p(qw.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
        ctypes.c_void_p(zr.data_ptr()), M, N, K, awq.config(g), ctypes.c_void_p(out.data_ptr()),
        2, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_call():
    import bit_weight_only_quantize_amd as awq
    torch = torch_mod()
    # first call: the batched-decode kernel (its split-K partials in the
    # static scratch); then bf16, K split 8 ways (partials and row factors);
    # then, smaller: fp16 split K; last: the GEMV (no scratch)
    shapes = [(16, 11008, 4096, 128, "f16"), (48, 6000, 4096, 128, "bf16"),
              (20, 3000, 2048, 64, "f16"), (3, 2000, 1024, 128, "f16")]
    for (M, N, K, g, dt) in shapes:
        W = wl.gen_weight(N, K, 170 + M)
        X = wl.gen_activation(M, K, 171 + M, 172, dt)
        qw, sc, zr = quantize_pack(W, QuantConfig(group_size=g))
        pd = (to_dev(qw), to_dev(sc), to_dev(zr))
        Xd = to_dev(X, bf16=(dt == "bf16"))
        say("noalloc", M, N, K, g, dt)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
        assert _call_noalloc(awq, Xd, pd, M, N, K, g, out) == 0, awq.lib.awq_last_error()
        need = awq.awq_linear_workspace_size(M, N, K, g, Xd.dtype)
        ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device=dev())
        ref = awq.awq_linear_ws(Xd, *pd, ws, group_size=g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        x64 = bf16_bits_to_f32(X).astype(np.float64) if dt == "bf16" else X.astype(np.float64)
        assert_close(out.cpu().numpy().astype(np.float64), linear64(x64, qw, sc, zr, g), "noalloc")
