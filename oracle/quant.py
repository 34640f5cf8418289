"""Oracle: group-wise asymmetric int4 quantizer, packing and dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
------------------
* w_bit = 4, q_group_size = 128, zero_point = True as the default config
  ("AWQ Advanced Usage Guide", sections "Group Size Configuration" and
  "Zero-Point Quantization"; the awq-quantization skill card's quant_config).
* A group is a run of consecutive weights that share one scale and one zero
  point; zero_point selects an asymmetric mapping with a zero point
  (ai.lansai.wang explainer, checkpoint-field table).
* All weights go to one uniform 4-bit grid; salient channels are protected by
  scaling, not by keeping an fp16 subset (ai.lansai.wang explainer, opening
  answer and its table of common claims).

What the pages leave open, and the reading taken here
-----------------------------------------------------
The pages print no quantizer formula and no packing layout.  The plainest
reading of "asymmetric uniform grid with a zero point" is min-max affine
quantisation with an integer zero point, written out below step by step:

  v      = fp32(s_k * W_nk)          (s_k = 1 when no scaling is given)
  lo, hi = min(min_g v, 0), max(max_g v, 0)   over the g values of one group
  s32    = (hi - lo) / 15            fp32 division
  s_h    = fp16_rne(max(s32, 2^-14)) the stored scale; codes use float(s_h)
  z      = clamp(rint(-lo / s_h), 0, 15)
  q      = clamp(rint(v / s_h) + z, 0, 15)
  deq    = (q - z) * s_h             exact in fp64

rint is round-half-to-even, every division is IEEE fp32 and correctly rounded.

Without a zero point ("Zero-Point Quantization": zero_point=False is the
symmetric variant; the pages give no formula), the plainest symmetric reading
is a grid centred on zero whose extremes are +-7 steps, so that the group's
largest magnitude lands exactly on a level:

  amax   = max_g |v|
  s32    = amax / 7                  fp32 division
  s_h    = fp16_rne(max(s32, 2^-14))
  q      = clamp(rint(v / s_h), -8, 7), stored as the code q + 8 (0..15)
  deq    = (code - 8) * s_h          (a fixed zero point of 8; no zeros array)

Packing (a layout of this project, not of the pages): qweight[n][c] is a u32
whose nibble p (bits 4p..4p+3) holds q[n][8c + ORDER[p]], ORDER =
(0, 2, 4, 6, 1, 3, 5, 7).  So nibble i and nibble i+4 of a word hold the pair
(k = 2i, k = 2i+1), one in each 16-bit half.

Parity pins (tests/test_oracle_quant.py): hand-worked groups with ties,
degenerate groups, the packed word of q = 0..7, pack/unpack round trip,
the round-trip error bound, brute-force nearest-level search on tiny groups,
power-of-two equivariance and permutation equivariance.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32
F16 = np.float16

#: Nibble p of a packed word holds the code of column 8c + ORDER[p].
ORDER = (0, 2, 4, 6, 1, 3, 5, 7)

#: Smallest stored scale: the smallest normal fp16 value.
SCALE_FLOOR = F32(2.0 ** -14)

#: Code of the symmetric grid's zero (codes are q + 8 for q in [-8, 7]).
SYM_ZERO = 8


@dataclass(frozen=True)
class QuantConfig:
    """Mirror of the pages' quant_config fields."""

    w_bit: int = 4
    group_size: int = 128
    zero_point: bool = True

    def check(self, K: int) -> None:
        if self.w_bit != 4:
            raise ValueError("only w_bit=4 is defined")
        if self.group_size <= 0 or K % self.group_size:
            raise ValueError("K must be a multiple of group_size")
        if K % 8:
            raise ValueError("K must be a multiple of 8")


def quantize_groups(W, group_size: int = 128, s=None, zero_point: bool = True):
    """Quantize W[N][K] (fp16) group-wise along K.

    Returns (q uint8 [N][K], scales fp16 [N][K/g], zeros uint8 [N][K/g]), or
    with zero_point=False the symmetric codes, the scales and None (every
    group's zero is SYM_ZERO).  ``s`` is an optional fp32 per-input-channel
    scale vector of length K; when given, the values quantized are
    fp32(s_k * W_nk) (the sW of Y=(X/s)(sW)).
    """
    W = np.asarray(W)
    if W.dtype != F16:
        raise TypeError("W must be float16")
    N, K = W.shape
    g = int(group_size)
    if K % g:
        raise ValueError("K must be a multiple of group_size")
    G = K // g

    # Step 1: the values to quantize, in fp32.
    v = W.astype(F32)
    if s is not None:
        s = np.asarray(s)
        if s.dtype != F32 or s.shape != (K,):
            raise TypeError("s must be float32 of shape (K,)")
        v = s[None, :] * v                      # one correctly-rounded fp32 product
    vg = v.reshape(N, G, g)

    if not zero_point:
        # Symmetric: the step puts the largest magnitude on level +-7.
        amax = np.abs(vg).max(axis=-1)
        s32 = amax / F32(7.0)
        s_h = np.maximum(s32, SCALE_FLOOR).astype(F16)
        sf = s_h.astype(F32)
        q = np.clip(np.rint(vg / sf[..., None]), F32(-8.0), F32(7.0)) + F32(SYM_ZERO)
        return q.reshape(N, K).astype(np.uint8), s_h, None

    # Step 2: the range of each group, widened to include 0.
    lo = np.minimum(vg.min(axis=-1), F32(0.0))
    hi = np.maximum(vg.max(axis=-1), F32(0.0))

    # Step 3: the step between the 16 levels, then its fp16 storage value.
    s32 = (hi - lo) / F32(15.0)
    s_h = np.maximum(s32, SCALE_FLOOR).astype(F16)
    sf = s_h.astype(F32)

    # Step 4: zero point and codes, rounded half-to-even, clamped to [0, 15].
    z = np.clip(np.rint(-lo / sf), F32(0.0), F32(15.0))
    q = np.clip(np.rint(vg / sf[..., None]) + z[..., None], F32(0.0), F32(15.0))

    return (q.reshape(N, K).astype(np.uint8), s_h, z.astype(np.uint8))


def pack_codes(q):
    """Pack uint8 codes q[N][K] (values 0..15) into u32 words [N][K/8]."""
    q = np.asarray(q)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    q8 = q.reshape(N, K // 8, 8).astype(np.uint32)
    out = np.zeros((N, K // 8), dtype=np.uint32)
    for p, col in enumerate(ORDER):
        out |= (q8[:, :, col] & np.uint32(0xF)) << np.uint32(4 * p)
    return out


def unpack_codes(qweight, K: int):
    """Inverse of :func:`pack_codes`."""
    qweight = np.asarray(qweight, dtype=np.uint32)
    N = qweight.shape[0]
    q = np.zeros((N, K // 8, 8), dtype=np.uint8)
    for p, col in enumerate(ORDER):
        q[:, :, col] = (qweight >> np.uint32(4 * p)) & np.uint32(0xF)
    return q.reshape(N, K)


def dequantize(q, scales, zeros, group_size: int = 128):
    """deq[n][k] = (q[n][k] - z[n][k//g]) * s_h[n][k//g], in fp64 (exact).
    zeros=None is the symmetric grid: z = SYM_ZERO for every group."""
    q = np.asarray(q)
    N, K = q.shape
    g = int(group_size)
    if zeros is None:
        zeros = np.full(np.asarray(scales).shape, SYM_ZERO, dtype=np.uint8)
    zr = np.repeat(np.asarray(zeros).astype(np.float64), g, axis=1)
    sc = np.repeat(np.asarray(scales).astype(np.float64), g, axis=1)
    return (q.astype(np.float64) - zr) * sc


def quantize_pack(W, cfg: QuantConfig = QuantConfig(), s=None):
    """Quantize and pack: returns (qweight u32 [N][K/8], scales f16 [N][G],
    zeros u8 [N][G] or None for the symmetric grid)."""
    W = np.asarray(W)
    cfg.check(W.shape[1])
    q, sc, zr = quantize_groups(W, cfg.group_size, s, cfg.zero_point)
    return pack_codes(q), sc, zr
