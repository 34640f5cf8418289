"""Shared helpers for the GPU parity tests (test infrastructure only)."""

import numpy as np

REL_FRO = 1e-3      # relative Frobenius error bound on floating-point outputs
MAX_ABS = 2e-2      # max absolute error bound per output element


def torch_mod():
    import torch
    return torch


def dev():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def to_dev(a, bf16=False):
    """numpy -> GPU tensor.  fp16 stays fp16; uint16 bf16 bit patterns become
    bfloat16 when bf16=True; uint32 becomes int32 bits."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(dev())
    return torch.from_numpy(a).to(dev())


def to_np(t):
    torch = torch_mod()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def out_to_f64(t):
    """GPU output tensor (fp16 / bf16 / fp32) -> fp64 numpy."""
    torch = torch_mod()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def assert_close(Y, Yref, what=""):
    err = Y - Yref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(Yref), 1e-300))
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    assert rel <= REL_FRO and mx <= MAX_ABS, f"{what}: rel_fro={rel:.3e} max_abs={mx:.3e}"
    return rel, mx


def say(*args):
    print("[gpu-case]", *args, flush=True)
