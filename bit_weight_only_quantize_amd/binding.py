"""ctypes binding of libawq355.so (argument marshalling only).

Every function here validates its tensors (dtype, shape, device), allocates
outputs (and, where asked, a workspace) with torch when the caller does not
pass them, and calls the C entry point of the same name on the current HIP
stream.  All computation happens in the library's HIP
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
AWQ_KERNEL_AUTO, AWQ_KERNEL_GEMV, AWQ_KERNEL_GEMM, AWQ_KERNEL_BATCHED = 0, 1, 2, 3
AWQ_EPILOGUE_NONE, AWQ_EPILOGUE_SILU_MUL = 0, 1
AWQ_MAX_PARTS = 4
AWQ_GEMV_MAX_M = 16
AWQ_BATCHED_MAX_M = 64

#: Every symbol include/awq355.h declares.
EXPORTS = (
    "awq_quantize_pack",
    "awq_dequantize",
    "awq_linear",
    "awq_linear_ex",
    "awq_linear_workspace_size",
    "awq_linear_ws",
    "awq_linear_noalloc",
    "awq_linear_fused_workspace_size",
    "awq_linear_fused",
    "awq_scale_search_workspace_size",
    "awq_scale_search",
    "awq_scale_search_workspace_size_ex",
    "awq_scale_search_ex",
    "awq_status_string",
    "awq_last_error",
    "awq_version",
)


class awq_config(ctypes.Structure):
    _fields_ = [("w_bit", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("zero_point", ctypes.c_int32)]


class awq_linear_part(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("N", ctypes.c_int64), ("Y", ctypes.c_void_p)]


class awq_search_options(ctypes.Structure):
    _fields_ = [("duo_scaling", ctypes.c_int32), ("apply_clip", ctypes.c_int32)]


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
    lib.awq_dequantize.argtypes = [vp, vp, vp, i64, i64, awq_config, vp, i32, vp]
    lib.awq_dequantize.restype = ctypes.c_int
    lib.awq_linear.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, vp]
    lib.awq_linear.restype = ctypes.c_int
    lib.awq_linear_ex.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, i32, vp,
                                  ctypes.c_size_t, vp]
    lib.awq_linear_ex.restype = ctypes.c_int
    lib.awq_linear_workspace_size.argtypes = [i64, i64, i64, awq_config, i32, i32]
    lib.awq_linear_workspace_size.restype = ctypes.c_size_t
    lib.awq_linear_ws.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32, vp,
                                  ctypes.c_size_t, vp]
    lib.awq_linear_ws.restype = ctypes.c_int
    pp = ctypes.POINTER(awq_linear_part)
    lib.awq_linear_fused_workspace_size.argtypes = [pp, i32, i64, i64, awq_config, i32, i32, i32]
    lib.awq_linear_fused_workspace_size.restype = ctypes.c_size_t
    lib.awq_linear_fused.argtypes = [vp, i32, pp, i32, i64, i64, awq_config, i32, vp, i32, i32,
                                     vp, ctypes.c_size_t, vp]
    lib.awq_linear_fused.restype = ctypes.c_int
    lib.awq_linear_noalloc.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, awq_config, vp, i32,
                                       vp]
    lib.awq_linear_noalloc.restype = ctypes.c_int
    lib.awq_scale_search_workspace_size.argtypes = [i64, i64, i64, awq_config, i32]
    lib.awq_scale_search_workspace_size.restype = ctypes.c_size_t
    lib.awq_scale_search.argtypes = [vp, vp, i64, i64, i64, awq_config,
                                     ctypes.POINTER(ctypes.c_double), i32, vp, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_double), vp, vp, vp, vp, vp]
    lib.awq_scale_search.restype = ctypes.c_int
    po = ctypes.POINTER(awq_search_options)
    lib.awq_scale_search_workspace_size_ex.argtypes = [i64, i64, i64, awq_config, i32, po]
    lib.awq_scale_search_workspace_size_ex.restype = ctypes.c_size_t
    lib.awq_scale_search_ex.argtypes = [vp, vp, i64, i64, i64, awq_config,
                                        ctypes.POINTER(ctypes.c_double), i32, po, vp,
                                        ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_double), vp, vp, vp, vp, vp, vp]
    lib.awq_scale_search_ex.restype = ctypes.c_int
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
#
# Every wrapper checks, before any C call: that each argument is a tensor of
# the expected dtype and shape (so no kernel can read or write past an
# allocation), then that all tensors sit on one GPU, contiguously.  Shape and
# dtype errors raise TypeError / ValueError even on machines without a GPU.

def _torch():
    import torch
    return torch


def _tensor(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _placed(*named):
    """All (tensor, name) pairs on one GPU and contiguous; returns the device."""
    dev = None
    for t, name in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} like the other tensors")
    return dev


def _ptr(t):
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


def empty_packed(N: int, K: int, group_size: int, device, zero_point: bool = True):
    """Allocate (qweight int32 [N][K/8], scales fp16 [N][K/g], zeros uint8 [N][K/g]);
    zeros is None for the symmetric grid (zero_point=False)."""
    torch = _torch()
    G = K // group_size
    return (torch.empty((N, K // 8), dtype=torch.int32, device=device),
            torch.empty((N, G), dtype=torch.float16, device=device),
            torch.empty((N, G), dtype=torch.uint8, device=device) if zero_point else None)


def _check_packed(qweight, scales, zeros, K, group_size):
    """Packed layer tensors for input width K (zeros None: the symmetric
    grid); returns N."""
    torch = _torch()
    if group_size <= 0 or K % group_size or K % 8:
        raise ValueError(f"K={K} must be a multiple of 8 and of group_size={group_size}")
    _tensor(qweight, "qweight", torch.int32)
    if qweight.dim() != 2:
        raise ValueError("qweight must be 2-D [N][K/8]")
    N = qweight.shape[0]
    _tensor(qweight, "qweight", shape=(N, K // 8))
    _tensor(scales, "scales", torch.float16, (N, K // group_size))
    if zeros is not None:
        _tensor(zeros, "zeros", torch.uint8, (N, K // group_size))
    return N


def _zp_ptr(zeros):
    return ctypes.c_void_p(0) if zeros is None else _ptr(zeros)


def awq_quantize_pack(W, group_size: int = 128, s=None, nonfinite_count=None, out=None,
                      zero_point: bool = True):
    """Quantize and pack W (fp16 [N][K], on the GPU).  Returns (qweight,
    scales, zeros); zeros is None for the symmetric grid (zero_point=False)."""
    torch = _torch()
    _tensor(W, "W", torch.float16)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N][K]")
    N, K = W.shape
    if group_size <= 0 or K % group_size or K % 8:
        raise ValueError(f"K={K} must be a multiple of 8 and of group_size={group_size}")
    if out is not None:
        qw, sc, zr = out
        if _check_packed(qw, sc, zr, K, group_size) != N:
            raise ValueError("out's packed tensors are not for N rows")
        if (zr is None) == bool(zero_point):
            raise ValueError("out's zeros must be a tensor exactly when zero_point is set")
    named = [(W, "W")]
    sp = ctypes.c_void_p(0)
    if s is not None:
        _tensor(s, "s", torch.float32, (K,))
        named.append((s, "s"))
        sp = _ptr(s)
    cp = ctypes.c_void_p(0)
    if nonfinite_count is not None:
        _tensor(nonfinite_count, "nonfinite_count", torch.int32)
        if nonfinite_count.numel() < 1:
            raise ValueError("nonfinite_count must hold one element")
        named.append((nonfinite_count, "nonfinite_count"))
        cp = _ptr(nonfinite_count)
    dev = _placed(*named)
    if out is None:
        qw, sc, zr = empty_packed(N, K, group_size, dev, zero_point)
    _placed((W, "W"), (qw, "qweight"), (sc, "scales"), *([] if zr is None else [(zr, "zeros")]))
    st = lib.awq_quantize_pack(_ptr(W), N, K, config(group_size, zero_point=zero_point), sp,
                               _ptr(qw), _ptr(sc), _zp_ptr(zr), cp, _stream(dev))
    check(st, "awq_quantize_pack")
    return qw, sc, zr


def awq_dequantize(qweight, scales, zeros, K: int, group_size: int = 128, out_dtype=None,
                   out=None):
    """(code - zero) * scale as a [N][K] tensor: float32 (exact, the default)
    or float16 (rounded once); zeros None for the symmetric grid."""
    torch = _torch()
    N = _check_packed(qweight, scales, zeros, K, group_size)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is not None:
        _tensor(out, "out", (torch.float16, torch.float32), (N, K))
        odt = out.dtype
    elif odt not in (torch.float16, torch.float32):
        raise TypeError(f"out_dtype {odt} is not float16 or float32")
    dev = _placed((qweight, "qweight"), (scales, "scales"),
                  *([] if zeros is None else [(zeros, "zeros")]))
    if out is None:
        out = torch.empty((N, K), dtype=odt, device=dev)
    _placed((qweight, "qweight"), (out, "out"))
    st = lib.awq_dequantize(_ptr(qweight), _ptr(scales), _zp_ptr(zeros), N, K,
                            config(group_size, zero_point=zeros is not None), _ptr(out),
                            _dtype_code(odt), _stream(dev))
    check(st, "awq_dequantize")
    return out


def _linear_args(X, qweight, scales, zeros, group_size, out_dtype, out):
    """Validate a linear call; returns (M, N, K, out, device)."""
    torch = _torch()
    _tensor(X, "X", (torch.float16, torch.bfloat16))
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    M, K = X.shape
    N = _check_packed(qweight, scales, zeros, K, group_size)
    ydt = (torch.float16, torch.bfloat16, torch.float32)
    if out is not None:
        _tensor(out, "out", ydt, (M, N))
    elif out_dtype is not None and out_dtype not in ydt:
        raise TypeError(f"out_dtype {out_dtype} is not float16, bfloat16 or float32")
    dev = _placed((X, "X"), (qweight, "qweight"), (scales, "scales"),
                  *([] if zeros is None else [(zeros, "zeros")]))
    if out is None:
        out = torch.empty((M, N), dtype=X.dtype if out_dtype is None else out_dtype, device=dev)
    _placed((X, "X"), (out, "out"))
    return M, N, K, out, dev


def awq_linear_workspace_size(M: int, N: int, K: int, group_size: int = 128,
                              x_dtype=None, kernel: int = AWQ_KERNEL_AUTO) -> int:
    """Workspace bytes the GEMM path needs (awq_linear_workspace_size); x_dtype
    is a torch dtype (default float16)."""
    torch = _torch()
    xd = AWQ_F16 if x_dtype is None or x_dtype == torch.float16 else _dtype_code(x_dtype)
    return int(lib.awq_linear_workspace_size(M, N, K, config(group_size), xd, int(kernel)))


def _workspace_arg(workspace, need, dev):
    torch = _torch()
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        if need == 0:
            return None
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is None:
        return None
    _tensor(workspace, "workspace")
    _placed((workspace, "workspace"))
    if workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    return workspace


def awq_linear_ex(X, qweight, scales, zeros, kernel: int = AWQ_KERNEL_AUTO,
                  group_size: int = 128, out_dtype=None, out=None, workspace="auto"):
    """Y = X * deq(W)^T with an explicit kernel choice (AWQ_KERNEL_*).

    ``workspace``: 'auto' (a torch-allocated buffer of
    awq_linear_workspace_size bytes when the call needs one), a uint8 tensor
    of at least that size (any contents), or None (the scratch-free plan, as
    awq_linear)."""
    if isinstance(workspace, str) and workspace != "auto":
        raise ValueError("workspace must be a tensor, None or 'auto'")
    if workspace is not None and not isinstance(workspace, str):
        _tensor(workspace, "workspace")
    M, N, K, out, dev = _linear_args(X, qweight, scales, zeros, group_size, out_dtype, out)
    need = awq_linear_workspace_size(M, N, K, group_size, X.dtype, kernel)
    ws = _workspace_arg(workspace, need, dev)
    st = lib.awq_linear_ex(_ptr(X), _dtype_code(X.dtype), _ptr(qweight), _ptr(scales),
                           _zp_ptr(zeros), M, N, K,
                           config(group_size, zero_point=zeros is not None), _ptr(out),
                           _dtype_code(out.dtype), int(kernel),
                           ctypes.c_void_p(0) if ws is None else _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(dev))
    check(st, "awq_linear_ex")
    return out


def awq_linear(X, qweight, scales, zeros, group_size: int = 128, out_dtype=None, out=None):
    """Y = X * deq(W)^T with no scratch memory (the C awq_linear): small M
    runs the GEMV, larger M the GEMM without a K split; bf16 activations on
    the GEMM path raise AwqError (use awq_linear_ex or awq_linear_ws)."""
    M, N, K, out, dev = _linear_args(X, qweight, scales, zeros, group_size, out_dtype, out)
    st = lib.awq_linear(_ptr(X), _dtype_code(X.dtype), _ptr(qweight), _ptr(scales),
                        _zp_ptr(zeros), M, N, K, config(group_size, zero_point=zeros is not None),
                        _ptr(out), _dtype_code(out.dtype), _stream(dev))
    check(st, "awq_linear")
    return out


def awq_linear_ws(X, qweight, scales, zeros, workspace, group_size: int = 128, out_dtype=None,
                  out=None):
    """awq_linear with a caller workspace (uint8 tensor of at least
    awq_linear_workspace_size bytes, any contents); the call allocates nothing."""
    M, N, K, out, dev = _linear_args(X, qweight, scales, zeros, group_size, out_dtype, out)
    ws = _workspace_arg(workspace, 0, dev)
    st = lib.awq_linear_ws(_ptr(X), _dtype_code(X.dtype), _ptr(qweight), _ptr(scales),
                           _zp_ptr(zeros), M, N, K,
                           config(group_size, zero_point=zeros is not None), _ptr(out),
                           _dtype_code(out.dtype),
                           ctypes.c_void_p(0) if ws is None else _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(dev))
    check(st, "awq_linear_ws")
    return out


def awq_linear_noalloc(X, qweight, scales, zeros, group_size: int = 128, out_dtype=None,
                       out=None):
    """awq_linear_ws with the library's static device scratch instead of a
    workspace: allocates nothing (pass `out` to allocate nothing here either).
    Calls that may overlap in time on one GPU must not be made."""
    M, N, K, out, dev = _linear_args(X, qweight, scales, zeros, group_size, out_dtype, out)
    st = lib.awq_linear_noalloc(_ptr(X), _dtype_code(X.dtype), _ptr(qweight), _ptr(scales),
                                _zp_ptr(zeros), M, N, K,
                                config(group_size, zero_point=zeros is not None), _ptr(out),
                                _dtype_code(out.dtype), _stream(dev))
    check(st, "awq_linear_noalloc")
    return out


def awq_linear_fused(X, parts, epilogue: str = "none", group_size: int = 128, out_dtype=None,
                     outs=None, kernel: int = AWQ_KERNEL_AUTO, workspace="auto"):
    """Several projections of one X (each part a (qweight, scales, zeros)
    tuple of the same K, group size and zero-point mode).  epilogue 'none'
    returns [X W_i^T for each part]; 'silu_mul' takes (gate, up) and returns
    silu(X Wg^T) * (X Wu^T).  `outs` optionally gives the output tensors (a
    list for 'none', one tensor for 'silu_mul')."""
    torch = _torch()
    if epilogue not in ("none", "silu_mul"):
        raise ValueError("epilogue must be 'none' or 'silu_mul'")
    if not 1 <= len(parts) <= AWQ_MAX_PARTS:
        raise ValueError(f"1 to {AWQ_MAX_PARTS} parts")
    pair = epilogue == "silu_mul"
    if pair and len(parts) != 2:
        raise ValueError("'silu_mul' takes exactly two parts (gate, up)")
    if isinstance(workspace, str) and workspace != "auto":
        raise ValueError("workspace must be a tensor, None or 'auto'")
    _tensor(X, "X", (torch.float16, torch.bfloat16))
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    M, K = X.shape
    Ns = [_check_packed(qw, sc, zr, K, group_size) for (qw, sc, zr) in parts]
    zp = parts[0][2] is not None
    if any((zr is not None) != zp for (_, _, zr) in parts):
        raise ValueError("all parts must share the zero-point mode")
    if pair and Ns[0] != Ns[1]:
        raise ValueError("gate and up must have the same N")
    ydt = (torch.float16, torch.bfloat16, torch.float32)
    odt = X.dtype if out_dtype is None else out_dtype
    if odt not in ydt:
        raise TypeError(f"out_dtype {odt} is not float16, bfloat16 or float32")
    if outs is not None:
        outl = [outs] if pair else list(outs)
        if len(outl) != (1 if pair else len(parts)):
            raise ValueError("one output per part ('none') or one H ('silu_mul')")
        for o, n in zip(outl, Ns[:len(outl)]):
            _tensor(o, "out", ydt, (M, n))
        if len({o.dtype for o in outl}) != 1:
            raise TypeError("every output must have the same dtype")
        odt = outl[0].dtype
    named = [(X, "X")]
    for i, (qw, sc, zr) in enumerate(parts):
        named += [(qw, f"parts[{i}].qweight"), (sc, f"parts[{i}].scales")]
        if zr is not None:
            named.append((zr, f"parts[{i}].zeros"))
    dev = _placed(*named)
    if outs is None:
        outl = [torch.empty((M, n), dtype=odt, device=dev) for n in (Ns[:1] if pair else Ns)]
    _placed(*[(o, "out") for o in outl])
    arr = (awq_linear_part * len(parts))()
    for i, (qw, sc, zr) in enumerate(parts):
        arr[i] = awq_linear_part(qw.data_ptr() if qw.numel() else None,
                                 sc.data_ptr() if sc.numel() else None,
                                 None if zr is None or not zr.numel() else zr.data_ptr(), Ns[i],
                                 None if pair else (outl[i].data_ptr() if outl[i].numel() else None))
    cfg = config(group_size, zero_point=zp)
    epi = AWQ_EPILOGUE_SILU_MUL if pair else AWQ_EPILOGUE_NONE
    xd = _dtype_code(X.dtype)
    need = int(lib.awq_linear_fused_workspace_size(arr, len(parts), M, K, cfg, xd, epi,
                                                   int(kernel)))
    if workspace is not None and not isinstance(workspace, str):
        _tensor(workspace, "workspace")
    ws = _workspace_arg(workspace, need, dev)
    H = outl[0] if pair else None
    st = lib.awq_linear_fused(_ptr(X), xd, arr, len(parts), M, K, cfg, epi,
                              ctypes.c_void_p(0) if H is None else _ptr(H), _dtype_code(odt),
                              int(kernel), ctypes.c_void_p(0) if ws is None else _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(dev))
    check(st, "awq_linear_fused")
    return H if pair else outl


def awq_scale_search_workspace_size(M: int, N: int, K: int, group_size: int = 128,
                                    n_alpha: int = 20, zero_point: bool = True,
                                    duo_scaling: bool = False, apply_clip: bool = False) -> int:
    cfg = config(group_size, zero_point=zero_point)
    opts = awq_search_options(int(bool(duo_scaling)), int(bool(apply_clip)))
    return int(lib.awq_scale_search_workspace_size_ex(M, N, K, cfg, n_alpha, ctypes.byref(opts)))


def awq_scale_search(X, W, group_size: int = 128, alphas=None, workspace=None, out=None,
                     zero_point: bool = True, duo_scaling: bool = False,
                     apply_clip: bool = False):
    """Alpha-grid scale search (awq_scale_search_ex).  Returns a dict with
    best_index, losses (numpy fp64), s (fp32 [K] tensor) and the packed
    weights for the chosen s (zeros None for the symmetric grid,
    zero_point=False); with apply_clip also clip_index (uint8 [N][K/g])."""
    torch = _torch()
    _tensor(X, "X", torch.float16)
    _tensor(W, "W", torch.float16)
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X must be [M][K] and W [N][K]")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W has {W.shape[1]} input channels, X has {K}")
    n_alpha = 20 if alphas is None else len(alphas)
    need = awq_scale_search_workspace_size(M, N, K, group_size, n_alpha, zero_point, duo_scaling,
                                           apply_clip)
    if need == 0:
        check(AWQ_ERR_INVALID_ARG, "awq_scale_search_workspace_size")
    if out is not None:
        qw, sc, zr = out
        if _check_packed(qw, sc, zr, K, group_size) != N:
            raise ValueError("out's packed tensors are not for N rows")
        if (zr is None) == bool(zero_point):
            raise ValueError("out's zeros must be a tensor exactly when zero_point is set")
    if workspace is not None:
        _tensor(workspace, "workspace")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {need} needed")
    dev = _placed((X, "X"), (W, "W"))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if out is None:
        qw, sc, zr = empty_packed(N, K, group_size, dev, zero_point)
    best_s = torch.empty(K, dtype=torch.float32, device=dev)
    _placed((X, "X"), (workspace, "workspace"), (qw, "qweight"), (sc, "scales"),
            *([] if zr is None else [(zr, "zeros")]))
    a_ptr = None
    if alphas is not None:
        a_arr = (ctypes.c_double * n_alpha)(*[float(a) for a in alphas])
        a_ptr = ctypes.cast(a_arr, ctypes.POINTER(ctypes.c_double))
    best = ctypes.c_int32(-1)
    losses = (ctypes.c_double * n_alpha)()
    opts = awq_search_options(int(bool(duo_scaling)), int(bool(apply_clip)))
    clip = (torch.empty((N, K // group_size), dtype=torch.uint8, device=dev)
            if apply_clip else None)
    st = lib.awq_scale_search_ex(_ptr(X), _ptr(W), M, N, K,
                                 config(group_size, zero_point=zero_point), a_ptr, n_alpha,
                                 ctypes.byref(opts), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 ctypes.byref(best), losses, _ptr(best_s), _ptr(qw), _ptr(sc),
                                 _zp_ptr(zr), ctypes.c_void_p(0) if clip is None else _ptr(clip),
                                 _stream(dev))
    check(st, "awq_scale_search_ex")
    res = {"best_index": int(best.value), "losses": np.array(losses[:], dtype=np.float64),
           "s": best_s, "qweight": qw, "scales": sc, "zeros": zr}
    if clip is not None:
        res["clip_index"] = clip
    return res
