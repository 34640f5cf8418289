"""ctypes binding of libawq355.so (argument marshalling only).

Every function here validates tensor placement, allocates outputs with torch
when the caller does not pass them, and calls the C entry point of the same
name on the current HIP stream.  All computation happens in the library's HIP
kernels; there is no fallback of any kind.  If the library is missing or
cannot be loaded, importing this module raises ImportError.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libawq355.so")

AWQ_OK = 0
AWQ_ERR_INVALID_ARG = 1
AWQ_ERR_UNSUPPORTED = 2
AWQ_ERR_WORKSPACE = 3
AWQ_ERR_HIP = 4
AWQ_ERR_NONFINITE = 5

AWQ_F16, AWQ_BF16, AWQ_F32 = 0, 1, 2
AWQ_KERNEL_AUTO, AWQ_KERNEL_GEMV, AWQ_KERNEL_GEMM = 0, 1, 2
AWQ_GEMV_MAX_M = 16

#: Every symbol include/awq355.h declares.
EXPORTS = (
    "awq_quantize_pack",
    "awq_linear",
    "awq_linear_ex",
    "awq_linear_workspace_size",
    "awq_linear_ws",
    "awq_scale_search_workspace_size",
    "awq_scale_search",
    "awq_status_string",
    "awq_last_error",
    "awq_version",
)


class awq_config(ctypes.Structure):
    _fields_ = [("w_bit", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("zero_point", ctypes.c_int32)]


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    # torch bundles its own HIP runtime under the same soname
    # (libamdhip64.so.7).  Importing torch first maps that runtime, and the
    # dynamic loader then resolves this library's dependency to the same copy,
    # so torch's streams and allocations are valid here.  Loading this library
    # first would map /opt/rocm's runtime and torch would add a second one.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bit_weight_only_quantize_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.awq_quantize_pack.argtypes = [vp, i64, i64, awq_config, vp, vp, vp, vp, vp, vp]
    lib.awq_quantize_pack.restype = ctypes.c_int
    lib.awq_linear.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, vp]
    lib.awq_linear.restype = ctypes.c_int
    lib.awq_linear_ex.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, i32, vp]
    lib.awq_linear_ex.restype = ctypes.c_int
    lib.awq_linear_workspace_size.argtypes = [i64, i64, i64, awq_config]
    lib.awq_linear_workspace_size.restype = ctypes.c_size_t
    lib.awq_linear_ws.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, vp,
                                  ctypes.c_size_t, vp]
    lib.awq_linear_ws.restype = ctypes.c_int
    lib.awq_scale_search_workspace_size.argtypes = [i64, i64, i64, awq_config, i32]
    lib.awq_scale_search_workspace_size.restype = ctypes.c_size_t
    lib.awq_scale_search.argtypes = [vp, vp, i64, i64, i64, awq_config,
                                     ctypes.POINTER(ctypes.c_double), i32, vp, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_double), vp, vp, vp, vp, vp]
    lib.awq_scale_search.restype = ctypes.c_int
    lib.awq_status_string.argtypes = [ctypes.c_int]
    lib.awq_status_string.restype = ctypes.c_char_p
    lib.awq_last_error.argtypes = []
    lib.awq_last_error.restype = ctypes.c_char_p
    lib.awq_version.argtypes = []
    lib.awq_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def config(group_size: int = 128, w_bit: int = 4, zero_point: bool = True) -> awq_config:
    return awq_config(int(w_bit), int(group_size), int(bool(zero_point)))


def check(status: int, what: str) -> None:
    if status != AWQ_OK:
        msg = lib.awq_last_error().decode() or lib.awq_status_string(status).decode()
        raise AwqError(status, f"{what}: {msg}")


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float16:
        return AWQ_F16
    if dt == torch.bfloat16:
        return AWQ_BF16
    if dt == torch.float32:
        return AWQ_F32
    raise TypeError(f"unsupported dtype {dt}")


def empty_packed(N: int, K: int, group_size: int, device):
    """Allocate (qweight int32 [N][K/8], scales fp16 [N][K/g], zeros uint8 [N][K/g])."""
    torch = _torch()
    G = K // group_size
    return (torch.empty((N, K // 8), dtype=torch.int32, device=device),
            torch.empty((N, G), dtype=torch.float16, device=device),
            torch.empty((N, G), dtype=torch.uint8, device=device))


def awq_quantize_pack(W, group_size: int = 128, s=None, nonfinite_count=None, out=None):
    """Quantize and pack W (fp16 [N][K], on the GPU).  Returns (qweight, scales, zeros)."""
    torch = _torch()
    if W.dtype != torch.float16 or W.dim() != 2:
        raise TypeError("W must be a 2-D float16 tensor")
    N, K = W.shape
    qw, sc, zr = out if out is not None else empty_packed(N, K, group_size, W.device)
    sp = ctypes.c_void_p(0)
    if s is not None:
        if s.dtype != torch.float32 or s.shape != (K,):
            raise TypeError("s must be float32 of shape (K,)")
        sp = _dev_ptr(s, "s")
    cp = ctypes.c_void_p(0)
    if nonfinite_count is not None:
        if nonfinite_count.dtype != torch.int32:
            raise TypeError("nonfinite_count must be int32")
        cp = _dev_ptr(nonfinite_count, "nonfinite_count")
    st = lib.awq_quantize_pack(_dev_ptr(W, "W"), N, K, config(group_size), sp,
                               _dev_ptr(qw, "qweight"), _dev_ptr(sc, "scales"),
                               _dev_ptr(zr, "zeros"), cp, _stream(W.device))
    check(st, "awq_quantize_pack")
    return qw, sc, zr


def awq_linear_ex(X, qweight, scales, zeros, kernel: int = AWQ_KERNEL_AUTO, group_size: int = 128,
                  out_dtype=None, out=None):
    """Y = X * deq(W)^T with an explicit kernel choice (AWQ_KERNEL_*)."""
    torch = _torch()
    if X.dim() != 2:
        raise TypeError("X must be 2-D")
    M, K = X.shape
    N = qweight.shape[0]
    if qweight.shape != (N, K // 8) or scales.shape != (N, K // group_size) or zeros.shape != scales.shape:
        raise ValueError("packed weight shapes do not match X and group_size")
    if out is None:
        odt = X.dtype if out_dtype is None else out_dtype
        out = torch.empty((M, N), dtype=odt, device=X.device)
    st = lib.awq_linear_ex(_dev_ptr(X, "X"), _dtype_code(X.dtype), _dev_ptr(qweight, "qweight"),
                           _dev_ptr(scales, "scales"), _dev_ptr(zeros, "zeros"), M, N, K,
                           config(group_size), _dev_ptr(out, "Y"), _dtype_code(out.dtype),
                           int(kernel), _stream(X.device))
    check(st, "awq_linear_ex")
    return out


def awq_linear(X, qweight, scales, zeros, group_size: int = 128, out_dtype=None, out=None):
    """Y = X * deq(W)^T; small M runs the GEMV kernel, larger M the GEMM."""
    return awq_linear_ex(X, qweight, scales, zeros, AWQ_KERNEL_AUTO, group_size, out_dtype, out)


def awq_linear_workspace_size(M: int, N: int, K: int, group_size: int = 128) -> int:
    return int(lib.awq_linear_workspace_size(M, N, K, config(group_size)))


def awq_linear_ws(X, qweight, scales, zeros, workspace, group_size: int = 128, out_dtype=None,
                  out=None):
    """awq_linear with a caller workspace (uint8 tensor of at least
    awq_linear_workspace_size bytes, any contents); the call allocates nothing."""
    torch = _torch()
    if X.dim() != 2:
        raise TypeError("X must be 2-D")
    M, K = X.shape
    N = qweight.shape[0]
    if qweight.shape != (N, K // 8) or scales.shape != (N, K // group_size) or zeros.shape != scales.shape:
        raise ValueError("packed weight shapes do not match X and group_size")
    if out is None:
        odt = X.dtype if out_dtype is None else out_dtype
        out = torch.empty((M, N), dtype=odt, device=X.device)
    wp = ctypes.c_void_p(0) if workspace is None else _dev_ptr(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.awq_linear_ws(_dev_ptr(X, "X"), _dtype_code(X.dtype), _dev_ptr(qweight, "qweight"),
                           _dev_ptr(scales, "scales"), _dev_ptr(zeros, "zeros"), M, N, K,
                           config(group_size), _dev_ptr(out, "Y"), _dtype_code(out.dtype), wp, wb,
                           _stream(X.device))
    check(st, "awq_linear_ws")
    return out


def awq_scale_search_workspace_size(M: int, N: int, K: int, group_size: int = 128,
                                    n_alpha: int = 20) -> int:
    return int(lib.awq_scale_search_workspace_size(M, N, K, config(group_size), n_alpha))


def awq_scale_search(X, W, group_size: int = 128, alphas=None, workspace=None, out=None):
    """Alpha-grid scale search.  Returns a dict with best_index, losses (numpy
    fp64), s (fp32 [K] tensor) and the packed weights for the chosen s."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0]
    n_alpha = 20 if alphas is None else len(alphas)
    need = awq_scale_search_workspace_size(M, N, K, group_size, n_alpha)
    if need == 0:
        check(AWQ_ERR_INVALID_ARG, "awq_scale_search_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    qw, sc, zr = out if out is not None else empty_packed(N, K, group_size, X.device)
    best_s = torch.empty(K, dtype=torch.float32, device=X.device)
    a_ptr = None
    if alphas is not None:
        a_arr = (ctypes.c_double * n_alpha)(*[float(a) for a in alphas])
        a_ptr = ctypes.cast(a_arr, ctypes.POINTER(ctypes.c_double))
    best = ctypes.c_int32(-1)
    losses = (ctypes.c_double * n_alpha)()
    st = lib.awq_scale_search(_dev_ptr(X, "X"), _dev_ptr(W, "W"), M, N, K, config(group_size),
                              a_ptr, n_alpha, _dev_ptr(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(),
                              ctypes.byref(best), losses, _dev_ptr(best_s, "best_s"),
                              _dev_ptr(qw, "qweight"), _dev_ptr(sc, "scales"),
                              _dev_ptr(zr, "zeros"), _stream(X.device))
    check(st, "awq_scale_search")
    return {"best_index": int(best.value), "losses": np.array(losses[:], dtype=np.float64),
            "s": best_s, "qweight": qw, "scales": sc, "zeros": zr}
