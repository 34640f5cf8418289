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


def weight_mean_abs(W):
    """wbar[k] = mean over output rows n of |W[n][k]| (fp16 W): the exact
    column sum divided by N, rounded once to fp64 (the same statistic as
    activation_mean_abs, taken over the weights)."""
    return activation_mean_abs(W)


def scale_vector(xbar, alpha: float, wbar=None):
    """One candidate scaling: fp32 s[k] from the fp64 statistic and one alpha.

    With ``wbar`` (duo scaling, "Calibration Parameters": duo_scaling scales
    by weights and activations; the page gives no formula): t_k = xbar_k^alpha
    / wbar_k^(1 - alpha), both floored at 2^-24, so alpha = 1 is the
    activation-only candidate and alpha = 0 the one that equalizes weight
    magnitudes.  Without it: t_k = xbar_k^alpha."""
    t = np.power(np.maximum(np.asarray(xbar, dtype=F64), STAT_FLOOR), F64(alpha))
    if wbar is not None:
        t = t / np.power(np.maximum(np.asarray(wbar, dtype=F64), STAT_FLOOR), F64(1.0) - F64(alpha))
    s = t / np.sqrt(t.max() * t.min())
    return s.astype(F32)


def scale_table(xbar, alphas=DEFAULT_ALPHAS, wbar=None):
    return np.stack([scale_vector(xbar, a, wbar) for a in alphas]).astype(F32)


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


def scale_search(X, W, cfg: QuantConfig = QuantConfig(), alphas=DEFAULT_ALPHAS, block: int = 1024,
                 duo_scaling: bool = False, apply_clip: bool = False):
    """Grid search over alpha.  Returns a dict with the chosen index, all losses,
    the statistic, the chosen fp32 scale vector and the packed weights for it
    (with apply_clip, the packed weights of the per-group clipping search,
    clip_search, on the chosen scaling; the losses are those of the unclipped
    candidates)."""
    X = np.asarray(X)
    W = np.asarray(W)
    cfg.check(W.shape[1])
    xbar = activation_mean_abs(X)
    wbar = weight_mean_abs(W) if duo_scaling else None
    Y_ref = reference_output(X, W, block)
    losses = np.empty(len(alphas), dtype=F64)
    best = None
    best_codes = None
    best_s = None
    for j, a in enumerate(alphas):
        s = scale_vector(xbar, a, wbar)
        L, codes = search_loss(X, W, s, cfg, Y_ref, block)
        losses[j] = L
        if best is None or L < losses[best]:       # strict: the first minimum wins
            best, best_codes, best_s = j, codes, s
    out = {"best_index": int(best), "losses": losses, "xbar": xbar, "wbar": wbar, "s": best_s}
    if apply_clip:
        clip = clip_search(X, W, best_s, cfg)
        out.update(qweight=pack_codes(clip["q"]), scales=clip["scales"], zeros=clip["zeros"],
                   clip_index=clip["clip_index"])
    else:
        q, sc, zr = best_codes
        out.update(qweight=pack_codes(q), scales=sc, zeros=zr)
    return out


# ---- weight clipping ----------------------------------------------------------------
#: Shrink factors of the clipping search: c_i = 1 - i/40, i = 0..19 (1 down to
#: 0.525), each rounded once to fp32.  ("Calibration Parameters" names
#: apply_clip, "Apply weight clipping", and no grid; this one mirrors the
#: alpha grid's 20 points and shrinks a range to at most about half.)
CLIP_GRID = (1.0 - np.arange(20, dtype=F64) / 40.0).astype(F32)


def quantize_group_clipped(v, c, group_size: int, zero_point: bool = True):
    """Quantize fp32 values v[..., g] (groups along the last axis) with each
    group's range shrunk by the fp32 factor c: the asymmetric range becomes
    [fp32(c * lo), fp32(c * hi)] (lo, hi as in quantize_groups), the symmetric
    one +-fp32(c * max|v|); then the step, zero point and codes follow
    quantize_groups exactly, so values beyond the shrunk range take the
    extreme codes.  c = 1 reproduces quantize_groups.  Returns (q, s_h, z)."""
    v = np.asarray(v, dtype=F32)
    c = F32(c)
    if zero_point:
        lo = np.minimum(v.min(axis=-1), F32(0.0)) * c
        hi = np.maximum(v.max(axis=-1), F32(0.0)) * c
        s32 = (hi - lo) / F32(15.0)
        s_h = np.maximum(s32, F32(2.0 ** -14)).astype(np.float16)
        sf = s_h.astype(F32)
        z = np.clip(np.rint(-lo / sf), F32(0.0), F32(15.0))
        q = np.clip(np.rint(v / sf[..., None]) + z[..., None], F32(0.0), F32(15.0))
        return q, s_h, z
    amax = np.abs(v).max(axis=-1) * c
    s32 = amax / F32(7.0)
    s_h = np.maximum(s32, F32(2.0 ** -14)).astype(np.float16)
    sf = s_h.astype(F32)
    q = np.clip(np.rint(v / sf[..., None]), F32(-8.0), F32(7.0)) + F32(8.0)
    return q, s_h, np.full(s_h.shape, F32(8.0))


def group_gram(A, group_size: int):
    """C[g] = A_g^T A_g in fp64 for the column groups of A (fp16 [M][K]): the
    products of fp16 values are exact in fp64."""
    A64 = np.asarray(A).astype(F64)
    M, K = A64.shape
    G = K // group_size
    return np.stack([A64[:, g * group_size:(g + 1) * group_size].T
                     @ A64[:, g * group_size:(g + 1) * group_size] for g in range(G)])


def clip_search(X, W, s, cfg: QuantConfig = QuantConfig(), grid=CLIP_GRID, all_errors=False):
    """Per (row n, group g), the shrink factor of `grid` whose quantization
    minimizes the group's contribution to the output error on the
    calibration inputs,
        E_c = || A_g (v_g - deq_c(v_g)) ||^2 = d^T C_g d,   d = v_g - deq_c(v_g),
    where A = fp16(X / s) is the activation the quantized layer sees, v =
    fp32(s * W) the weights it quantizes and C_g = A_g^T A_g (the objective of
    "How AWQ Works", restricted to one group of one output).  d is exact in
    fp64, E in fp64; the first minimum wins.  Returns dict(clip_index u8
    [N][G], q u8 [N][K], scales fp16 [N][G], zeros u8 [N][G] or None)."""
    W = np.asarray(W)
    N, K = W.shape
    g = cfg.group_size
    G = K // g
    s = np.asarray(s, dtype=F32)
    v = (s[None, :] * W.astype(F32)).reshape(N, G, g)
    C = group_gram(scaled_activation(X, s), g)
    best_E = np.full((N, G), np.inf)
    best_i = np.zeros((N, G), dtype=np.uint8)
    q_out = np.zeros((N, G, g), dtype=F32)
    s_out = np.zeros((N, G), dtype=np.float16)
    z_out = np.zeros((N, G), dtype=F32)
    errors = []
    for i, c in enumerate(np.asarray(grid, dtype=F32)):
        q, s_h, z = quantize_group_clipped(v, c, g, cfg.zero_point)
        deq = (q.astype(F64) - z.astype(F64)[..., None]) * s_h.astype(F64)[..., None]
        d = v.astype(F64) - deq
        # E[n][g] = d[n,g]^T C[g] d[n,g]
        E = np.stack([np.sum((d[:, gi] @ C[gi]) * d[:, gi], axis=1) for gi in range(G)], axis=1)
        if all_errors:
            errors.append(E)
        take = E < best_E                          # strict: the first minimum wins
        best_E = np.where(take, E, best_E)
        best_i[take] = i
        q_out[take] = q[take]
        s_out[take] = s_h[take]
        z_out[take] = z[take]
    out = {"clip_index": best_i, "q": q_out.reshape(N, K).astype(np.uint8), "scales": s_out,
           "zeros": z_out.astype(np.uint8) if cfg.zero_point else None, "errors": best_E}
    if all_errors:
        out["all_errors"] = np.stack(errors)
    return out
