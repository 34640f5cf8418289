"""Seeded synthetic inputs for the W4A16 layer and the scale search.

This module holds shapes, seeds and random draws only: no quantization,
dequantization, matmul or search arithmetic.  Both the CPU oracle tests and
the GPU path draw their inputs from here, and nothing else is shared.

Recipe (every draw is NumPy ``default_rng`` / PCG64, made in float64, scaled,
then cast round-to-nearest-even to fp16, or to bf16 through fp32):

* weights   W[n][k] = 0.02 * Z[n][k], Z ~ N(0, 1); for the decode shapes each
  output row n is further multiplied by exp(0.3 * G[n]), G ~ N(0, 1)
  (a LogNormal(0, 0.3) per-row magnitude).
* activations X[m][k] ~ N(0, 1) with round(0.01 * K) input channels, drawn
  without replacement, multiplied by 20 (the ~1% salient channels the pages
  describe: gtnt.cn report, section 一; skill card, "AWQ vs alternatives").
* seeds: the tiny layer uses W=0, X=1, outlier indices=2; every other case uses
  base = 100 * config + 10 * shape and W=base, X=base+1, outliers=base+2,
  row factors=base+3.

The pages calibrate on text corpora and evaluate on model benchmarks; neither
datasets nor trained weights are available, so these synthetic tensors stand in
for calibration activations (4096 tokens = 8 x 512, the pages'
max_calib_seq_len) and for the projection weights of 7B / 13B / 70B-class
layers.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

W_SIGMA = 0.02
ROW_SIGMA = 0.3
OUTLIER_GAIN = 20.0
_CHUNK_ROWS = 1024


def n_outliers(K: int) -> int:
    return int(round(0.01 * K))


def outlier_channels(K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, size=n_outliers(K), replace=False))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def gen_weight(N: int, K: int, seed: int, row_seed: int | None = None) -> np.ndarray:
    """fp16 W[N][K]; with ``row_seed`` each row carries a LogNormal(0, 0.3) factor."""
    rng = np.random.default_rng(seed)
    out = np.empty((N, K), dtype=np.float16)
    row = None
    if row_seed is not None:
        row = np.exp(ROW_SIGMA * np.random.default_rng(row_seed).standard_normal(N))
    for n0 in range(0, N, _CHUNK_ROWS):
        n1 = min(N, n0 + _CHUNK_ROWS)
        z = rng.standard_normal((n1 - n0, K)) * W_SIGMA
        if row is not None:
            z *= row[n0:n1, None]
        out[n0:n1] = z.astype(np.float16)
    return out


def gen_activation(M: int, K: int, seed: int, outlier_seed: int, dtype: str = "f16") -> np.ndarray:
    """X[M][K] ~ N(0,1) with 1% of channels x20.

    ``dtype`` 'f16' returns float16; 'bf16' returns the uint16 bf16 bit patterns.
    """
    rng = np.random.default_rng(seed)
    idx = outlier_channels(K, outlier_seed)
    gain = np.ones(K)
    gain[idx] = OUTLIER_GAIN
    if dtype == "f16":
        out = np.empty((M, K), dtype=np.float16)
    elif dtype == "bf16":
        out = np.empty((M, K), dtype=np.uint16)
    else:
        raise ValueError(dtype)
    for m0 in range(0, M, _CHUNK_ROWS):
        m1 = min(M, m0 + _CHUNK_ROWS)
        x = rng.standard_normal((m1 - m0, K)) * gain[None, :]
        if dtype == "f16":
            out[m0:m1] = x.astype(np.float16)
        else:
            out[m0:m1] = f32_to_bf16_bits(x.astype(np.float32))
    return out


#: Activation distributions with a non-zero mean (stress inputs for the
#: linear layer's accuracy: outputs grow with the mean, and so do the rounding
#: errors of any kernel that rounds dequantized weights or cancels large sums).
SHIFTED_KINDS = ("abs", "mean3", "mean40")


def gen_activation_shifted(M: int, K: int, seed: int, kind: str, dtype: str = "f16") -> np.ndarray:
    """X[M][K] = |N(0,1)| ('abs'), N(3,1) ('mean3') or N(0,1) + 40 ('mean40'),
    without outlier channels; 'f16' returns float16, 'bf16' uint16 bf16 bits."""
    z = np.random.default_rng(seed).standard_normal((M, K))
    if kind == "abs":
        x = np.abs(z)
    elif kind == "mean3":
        x = z + 3.0
    elif kind == "mean40":
        x = z + 40.0
    else:
        raise ValueError(kind)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


@dataclass(frozen=True)
class Case:
    """One layer shape with its seeds."""

    name: str
    config: int           # 1..5, the workload family
    M: int
    K: int
    N: int
    group_size: int = 128
    x_dtype: str = "f16"
    w_seed: int = 0
    x_seed: int = 1
    outlier_seed: int = 2
    row_seed: int | None = None
    tags: tuple = field(default=())

    def weight(self) -> np.ndarray:
        return gen_weight(self.N, self.K, self.w_seed, self.row_seed)

    def activation(self, M: int | None = None) -> np.ndarray:
        return gen_activation(self.M if M is None else M, self.K, self.x_seed,
                              self.outlier_seed, self.x_dtype)

    @property
    def weight_bytes(self) -> int:
        """Packed weights + fp16 scales + u8 zeros, the bytes a linear call must read."""
        G = self.K // self.group_size
        return self.N * self.K // 2 + 3 * self.N * G

    @property
    def io_bytes(self) -> int:
        """Bytes a linear call must move to and from HBM at least: the packed
        layer plus the fp16 activations read and the fp16 outputs written."""
        return self.weight_bytes + 2 * self.M * self.K + 2 * self.M * self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _seeded(config: int, shape: int) -> dict:
    base = 100 * config + 10 * shape
    return dict(w_seed=base, x_seed=base + 1, outlier_seed=base + 2)


def tiny_cases():
    return [Case(f"tiny_m{M}", 1, M, 512, 512, 128, "f16", 0, 1, 2) for M in (1, 8)]


GEMV_SHAPES = ((4096, 4096), (4096, 11008), (11008, 4096))       # (K, N)
GEMM_SHAPES = ((5120, 13824), (13824, 5120))
PREFILL_SHAPES = ((8192, 28672), (28672, 8192))


def gemv_cases(Ms=(1, 4)):
    out = []
    for i, (K, N) in enumerate(GEMV_SHAPES):
        sd = _seeded(2, i)
        for M in Ms:
            out.append(Case(f"gemv_k{K}_n{N}_m{M}", 2, M, K, N, 128, "f16",
                            row_seed=sd["w_seed"] + 3, **sd))
    return out


def gemm_cases(Ms=(16, 64, 256), groups=(64, 128)):
    out = []
    for i, (K, N) in enumerate(GEMM_SHAPES):
        sd = _seeded(3, i)
        for g in groups:
            for M in Ms:
                out.append(Case(f"gemm_k{K}_n{N}_m{M}_g{g}", 3, M, K, N, g, "f16", **sd))
    return out


def prefill_cases(dtypes=("f16", "bf16")):
    out = []
    for i, (K, N) in enumerate(PREFILL_SHAPES):
        sd = _seeded(4, i)
        for dt in dtypes:
            out.append(Case(f"prefill_k{K}_n{N}_{dt}", 4, 4096, K, N, 128, dt, **sd))
    return out


def search_case():
    return Case("search_4096", 5, 4096, 4096, 4096, 128, "f16", **_seeded(5, 0))


def all_cases():
    return tiny_cases() + gemv_cases() + gemm_cases() + prefill_cases() + [search_case()]
