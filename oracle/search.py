"""Oracle: activation statistic, equivalent scaling and the alpha-grid search.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
------------------
* Y = XW = (X/s)(sW) with s positive and per input channel; before
  quantization the two sides are equal (ai.lansai.wang explainer, section
  "AWQ 的四步链路", first paragraph).
* The objective L(s) = ||Q(W*s)(s^-1*X) - W*X|| ("AWQ Advanced Usage Guide",
  section "How AWQ Works", "Core formula").
* Salient channels are found from activation magnitudes on calibration inputs
  and receive the larger scaling factors (the same section, steps 1-2; gtnt.cn
  report, section 一).
* The search evaluates the reconstruction error of candidate scalings and keeps
  the best (ai.lansai.wang explainer, four-stage table, "搜索缩放" row).

What the pages leave open, and the reading taken here
-----------------------------------------------------
* Statistic: xbar_k = (1/M) sum_m |X_mk|: the exact sum (every fp16 magnitude
  is an integer number of units of 2^-24, below 2^40, so the sum is an exact
  integer for M < 2^24 and does not depend on summation order), divided by M
  and rounded once to fp64.
* Candidate scalings: s_k = t_k / sqrt(max_k t * min_k t), t_k =
  max(xbar_k, 2^-24)^alpha, alpha on the grid {0, 0.05, ..., 0.95}, computed
  in fp64 and rounded once to fp32.  alpha = 0 gives s = 1 exactly (plain
  round-to-nearest quantization).  The normalisation only centres s on 1 in log
  scale; L is unchanged by a power-of-two factor on s.
* Scaled activation: A = fp16(fp32(X) / s) (the 1/s is folded into the
  preceding op, so the quantized layer consumes fp16 activations).
* Norm: the squared Frobenius norm, summed in fp64, of Y_ref - A*deq^T with
  Y_ref = X*W^T exact in fp64 (the argmin equals that of the plain norm).
* Tie-break: the smallest alpha index that attains the minimum.

Parity pins (tests/test_oracle_search.py): xbar closed forms, a two-channel
s-table in closed form, s(alpha=0) = 1 and the codes then equal the unscaled
quantizer, the pre-quantization identity (X/s)(sW)^T = XW^T to 1e-13, L = 0 on
a lossless grid, L bit-identical under s -> 2s, L exactly x4 under X -> 2X, a
pure-Python-loop loss on tiny inputs, and L(alpha*) <= L(0).

Parity unpinned: host and device fp64 pow are different implementations; s is
compared bitwise at run time (agreement after the fp32 rounding fails only if
the fp64 results straddle an fp32 rounding boundary).
"""

from __future__ import annotations

import numpy as np

from .quant import QuantConfig, dequantize, quantize_groups, pack_codes

F16 = np.float16
F32 = np.float32
F64 = np.float64

#: alpha_j = j / 20, j = 0..19, in fp64.
DEFAULT_ALPHAS = np.arange(20, dtype=F64) / 20.0

#: Floor applied to the statistic before the power (keeps t > 0).
STAT_FLOOR = 2.0 ** -24


def activation_mean_abs(X):
    """xbar[k] = mean over rows m of |X[m][k]|: the exact column sum divided by
    M, rounded once to fp64 (X fp16, M < 2^24)."""
    X = np.asarray(X)
    if X.dtype != F16:
        raise TypeError("X must be float16")
    M = X.shape[0]
    if not 0 < M < 2 ** 24:
        raise ValueError("M must be in [1, 2^24)")
    # |x| * 2^24 is an integer below 2^40 and exact in fp64; the uint64 column
    # sums stay below 2^64.
    units = (np.abs(X.astype(F64)) * 2.0 ** 24).astype(np.uint64)
    sums = units.sum(axis=0, dtype=np.uint64)
    # Python's int / int is the correctly rounded quotient; * 2^-24 is exact.
    return np.array([(int(t) / M) * 2.0 ** -24 for t in sums], dtype=F64)


def scale_vector(xbar, alpha: float):
    """One candidate scaling: fp32 s[k] from the fp64 statistic and one alpha."""
    t = np.power(np.maximum(np.asarray(xbar, dtype=F64), STAT_FLOOR), F64(alpha))
    s = t / np.sqrt(t.max() * t.min())
    return s.astype(F32)


def scale_table(xbar, alphas=DEFAULT_ALPHAS):
    return np.stack([scale_vector(xbar, a) for a in alphas]).astype(F32)


def scaled_activation(X, s):
    """A = fp16(fp32(X) / s), the activation with 1/s folded in."""
    return (np.asarray(X).astype(F32) / np.asarray(s, dtype=F32)[None, :]).astype(F16)


def reference_output(X, W, block: int = 1024):
    """Y_ref = X * W^T in fp64 (blocked over output columns to bound memory)."""
    X64 = np.asarray(X).astype(F64)
    W = np.asarray(W)
    N = W.shape[0]
    out = np.empty((X64.shape[0], N), dtype=F64)
    for n0 in range(0, N, block):
        out[:, n0:n0 + block] = X64 @ W[n0:n0 + block].astype(F64).T
    return out


def search_loss(X, W, s, cfg: QuantConfig = QuantConfig(), Y_ref=None, block: int = 1024):
    """L(s) = sum (Y_ref - A * deq(Q(sW))^T)^2 in fp64, A = fp16(X/s).

    Returns (L, (q, scales, zeros)) so the caller can keep the codes of the
    winning candidate.
    """
    W = np.asarray(W)
    if Y_ref is None:
        Y_ref = reference_output(X, W, block)
    q, sc, zr = quantize_groups(W, cfg.group_size, s, cfg.zero_point)
    A64 = scaled_activation(X, s).astype(F64)
    N = W.shape[0]
    total = F64(0.0)
    for n0 in range(0, N, block):
        deq = dequantize(q[n0:n0 + block], sc[n0:n0 + block],
                         None if zr is None else zr[n0:n0 + block], cfg.group_size)
        E = Y_ref[:, n0:n0 + block] - A64 @ deq.T
        total += np.sum(E * E)
    return float(total), (q, sc, zr)


def scale_search(X, W, cfg: QuantConfig = QuantConfig(), alphas=DEFAULT_ALPHAS, block: int = 1024):
    """Grid search over alpha.  Returns a dict with the chosen index, all losses,
    the statistic, the chosen fp32 scale vector and the packed weights for it."""
    X = np.asarray(X)
    W = np.asarray(W)
    cfg.check(W.shape[1])
    xbar = activation_mean_abs(X)
    Y_ref = reference_output(X, W, block)
    losses = np.empty(len(alphas), dtype=F64)
    best = None
    best_codes = None
    best_s = None
    for j, a in enumerate(alphas):
        s = scale_vector(xbar, a)
        L, codes = search_loss(X, W, s, cfg, Y_ref, block)
        losses[j] = L
        if best is None or L < losses[best]:       # strict: the first minimum wins
            best, best_codes, best_s = j, codes, s
    q, sc, zr = best_codes
    return {
        "best_index": int(best),
        "losses": losses,
        "xbar": xbar,
        "s": best_s,
        "qweight": pack_codes(q),
        "scales": sc,
        "zeros": zr,
    }
