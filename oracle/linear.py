"""Oracle: the W4A16 linear layer Y = X * deq(W)^T in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe the quantized linear layer as weight-only: activations stay
in 16-bit floating point and only the weights are 4-bit ("W4A16"), the weights
being dequantized for the product (ai.lansai.wang explainer, table of common
claims: activation-aware does not mean 4-bit activations; the skill card's
"WQLinear Kernel Variants": GEMM and GEMV compute the same layer).

Definition written out: Y[m][n] = sum_k X[m][k] * (q[n][k] - z[n][k//g]) * s[n][k//g].
Every term is exact in fp64 and the sum is a single fp64 BLAS product, so the
result is the exact value up to fp64 rounding.

Parity pins (tests/test_oracle_linear.py): a one-hot X reproduces a column of
the dequantized matrix exactly; a pure-Python triple loop agrees to 1e-12
relative on small shapes; Y of a lossless grid equals X*W^T exactly.
"""

from __future__ import annotations

import numpy as np

from .quant import dequantize, unpack_codes


def _deq_from_packed(qweight, scales, zeros, K, group_size):
    q = unpack_codes(qweight, K)
    return dequantize(q, scales, zeros, group_size)


def linear64(X, qweight, scales, zeros, group_size: int = 128, rows=None, cols=None):
    """fp64 Y = X * deq^T.  X is any float array [M][K] (fp16, fp32, ...).

    ``rows`` / ``cols`` optionally select a subset of output rows (m) and
    columns (n); only those entries are computed (used for sampled checks of
    layers too large to evaluate whole).
    """
    X = np.asarray(X)
    K = X.shape[1]
    qweight = np.asarray(qweight)
    scales = np.asarray(scales)
    zeros = None if zeros is None else np.asarray(zeros)
    if cols is not None:
        cols = np.asarray(cols)
        qweight, scales = qweight[cols], scales[cols]
        zeros = None if zeros is None else zeros[cols]
    if rows is not None:
        X = X[np.asarray(rows)]
    deq = _deq_from_packed(qweight, scales, zeros, K, group_size)
    return X.astype(np.float64) @ deq.T


def linear_naive(X, q, scales, zeros, group_size: int = 128):
    """Pure-Python loops over (m, n, k); for tiny shapes only (zeros=None:
    the symmetric grid, zero 8)."""
    X = np.asarray(X).astype(np.float64)
    M, K = X.shape
    N = q.shape[0]
    g = group_size
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                grp = k // g
                z = 8.0 if zeros is None else float(zeros[n][grp])
                w = (float(q[n][k]) - z) * float(scales[n][grp])
                acc += float(X[m][k]) * w
            Y[m][n] = acc
    return np.array(Y, dtype=np.float64)


def silu64(x):
    """silu(x) = x * sigmoid(x) = x / (1 + e^-x), in fp64.

    The fused gate/up projections ("AWQ Advanced Usage Guide", "Layer
    Fusion": "Gate and Up projections fused") feed the MLP's gated activation,
    silu(gate) * up; the page names the fusion, not the activation, and the
    plainest reading is the SiLU-gated MLP of the Llama-class models the pages
    quantize."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def gate_up_silu64(X, gate, up, group_size: int = 128):
    """silu(X * deq(Wg)^T) * (X * deq(Wu)^T) in fp64; gate and up are
    (qweight, scales, zeros) of the same [N][K]."""
    return silu64(linear64(X, *gate, group_size)) * linear64(X, *up, group_size)
