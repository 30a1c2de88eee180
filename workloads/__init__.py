"""Seeded synthetic inputs for the W4A16 group-quantized linear.

This module is the only code shared by the CPU oracle and the HIP path.  It
draws weights and activations and nothing else: it holds none of the
quantizer's, packer's or linear layer's arithmetic.  Planting input outliers
(multiplying chosen entries by a constant) and casting activations to fp16 are
part of building the input, not of the method.

The shapes follow the layers the pages talk about (Llama-style MLP
projections, 7B/8B/70B) and the group size of 128 input channels that the
pages use throughout (DeepCompressor README, perplexity table rows
"W4A16 g128"; SqueezeLLM explainer, section 5.3).  The dense-and-sparse
configurations take their sparsity ratios (0.45 % and 0.05 %) from the
SqueezeLLM explainer, section 2.2.

Draw order for one configuration, from ``numpy.random.default_rng(seed)``
(PCG64):

1. ``W = standard_normal((N, K), float32) * float32(sigma)``
2. planted weight outliers: ``choice(N*K, n_planted, replace=False)`` flat
   positions, each multiplied by ``float32(w_outlier_mult)``
3. ``x = standard_normal((M, K), float32)``
4. activation outlier channels: ``choice(K, n_channels, replace=False)``,
   columns multiplied by ``float32(x_outlier_mult)``
5. ``x.astype(float16)`` (round to nearest even)

Config 5 draws W alone from seed 5000 and each ``x`` of height M from its
own ``default_rng(5000 + M)``, so the M sweep shares one weight matrix.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    Ms: Tuple[int, ...]
    N: int
    K: int
    sigma: float
    # planted weight outliers: count = floor(w_outlier_ppm * N * K / 1e6)
    w_outlier_ppm: int = 0
    w_outlier_mult: float = 1.0
    # sparse outlier branch: sparse_k = floor(sparse_ppm * N * K / 1e6)
    sparse_ppm: int = 0
    # activation outlier channels
    x_outlier_channels: int = 0
    x_outlier_mult: float = 1.0
    separate_x_seeds: bool = False
    group: int = GROUP

    @property
    def seed(self) -> int:
        return 1000 * self.index

    @property
    def n_planted(self) -> int:
        return (self.w_outlier_ppm * self.N * self.K) // 1_000_000

    @property
    def sparse_k(self) -> int:
        return (self.sparse_ppm * self.N * self.K) // 1_000_000


CONFIGS = {
    1: Config(1, "tiny", (1,), 512, 512, 0.02, w_outlier_ppm=5000, w_outlier_mult=20.0),
    2: Config(2, "decode_7b_up_proj", (1,), 11008, 4096, 0.02,
              w_outlier_ppm=1000, w_outlier_mult=20.0),
    3: Config(3, "batched_decode_dense_sparse", (16,), 4096, 4096, 0.02, sparse_ppm=4500),
    4: Config(4, "prefill_llama3_8b_mlp", (2048,), 14336, 4096, 0.02,
              x_outlier_channels=8, x_outlier_mult=30.0),
    5: Config(5, "down_proj_70b_sweep", (1, 8, 64, 512), 8192, 28672, 0.015,
              sparse_ppm=500, separate_x_seeds=True),
}


# Outlier density of the dense-and-sparse decomposition (0.45 % of the weights, the
# batched-decode layer's) given to a layer whose configuration has none, to time and
# check the prefill GEMM with a CSR term.
SPARSE_PPM_DENSE_AND_SPARSE = 4500


def _draw_weights(rng: np.random.Generator, cfg: Config, N: int, K: int) -> np.ndarray:
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(cfg.sigma)
    n_planted = (cfg.w_outlier_ppm * N * K) // 1_000_000
    if n_planted:
        pos = rng.choice(N * K, n_planted, replace=False)
        flat = W.reshape(-1)
        flat[pos] *= np.float32(cfg.w_outlier_mult)
    return W


def _draw_x(rng: np.random.Generator, cfg: Config, M: int, K: int) -> np.ndarray:
    x = rng.standard_normal((M, K), dtype=np.float32)
    if cfg.x_outlier_channels:
        ch = rng.choice(K, cfg.x_outlier_channels, replace=False)
        x[:, ch] *= np.float32(cfg.x_outlier_mult)
    return x.astype(np.float16)


def make(index: int, M: int | None = None, N: int | None = None, K: int | None = None):
    """Return ``(W float32 [N,K], x float16 [M,K], cfg)`` for a configuration.

    ``N``/``K`` overrides shrink a configuration while keeping its value
    recipe (used for small parity cases); ``M`` defaults to the first M of
    the configuration.
    """
    cfg = CONFIGS[index]
    M = cfg.Ms[0] if M is None else M
    N = cfg.N if N is None else N
    K = cfg.K if K is None else K
    if cfg.separate_x_seeds:
        W = _draw_weights(np.random.default_rng(cfg.seed), cfg, N, K)
        x = _draw_x(np.random.default_rng(cfg.seed + M), cfg, M, K)
    else:
        rng = np.random.default_rng(cfg.seed)
        W = _draw_weights(rng, cfg, N, K)
        x = _draw_x(rng, cfg, M, K)
    return W, x, cfg


def sparse_k_for(cfg: Config, N: int, K: int) -> int:
    return (cfg.sparse_ppm * N * K) // 1_000_000


def random_weights(seed: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """Plain N(0, sigma) float32 weights, for edge-case shapes."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(sigma)
    return W


def random_x(seed: int, M: int, K: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) activations cast to fp16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x.astype(np.float16)


def integer_case(seed: int, M: int, N: int, K: int, nnz_per_row: int = 3, group: int = GROUP):
    """Inputs on which every product and partial sum is exact in fp32.

    Codes q in [0, 15], integer zero-points z in [0, 15], power-of-two scales
    (2^-4 .. 2^-1), activations in {-4..4} and integer sparse values in
    [-8, 8] \\ {0} at distinct, ascending columns.  Returned as the stored
    metadata directly (codes, fp16 scale/zero bit patterns, CSR), i.e. what a
    quantizer would have produced.
    """
    rng = np.random.default_rng(seed)
    G = K // group
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, G)).astype(np.float16)
    s = (2.0 ** -rng.integers(1, 5, size=(N, G))).astype(np.float16)
    x = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    cols, vals, row_ptr = [], [], [0]
    for _ in range(N):
        c = np.sort(rng.choice(K, nnz_per_row, replace=False)).astype(np.int32)
        v = rng.integers(1, 9, size=nnz_per_row) * rng.choice([-1, 1], size=nnz_per_row)
        cols.append(c)
        vals.append(v.astype(np.float16))
        row_ptr.append(row_ptr[-1] + nnz_per_row)
    row_ptr = np.asarray(row_ptr, dtype=np.int32)
    col = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    val = np.concatenate(vals) if vals else np.zeros(0, np.float16)
    return x, q, s, z, row_ptr, col, val


def lowrank_factors(seed: int, r: int, N: int, K: int, sigma_up: float = 0.2):
    """Random fp16 factors of a rank-r branch: L1 [r, K] ~ N(0, 1/K) (so that
    x . L1^T stays of unit size for unit activations) and L2 [N, r] ~ N(0,
    sigma_up^2).  No rank or factor values are given by the pages; these only
    give the branch a size comparable to the dense product."""
    rng = np.random.default_rng(seed)
    L1 = (rng.standard_normal((r, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))).astype(np.float16)
    L2 = (rng.standard_normal((N, r), dtype=np.float32) * np.float32(sigma_up)).astype(np.float16)
    return L1, L2


def integer_lowrank_factors(seed: int, r: int, N: int, K: int, nnz_per_row: int = 256):
    """Integer factors for the exact case: L1 [r, K] in {-1, 0, 1} with at most
    nnz_per_row non-zeros per row and L2 [N, r] in {-2..2}.  With activations in
    {-4..4} and nnz_per_row <= 256, every |x . L1^T| <= 1024 is an integer that
    fp16 holds exactly, and every partial sum of the branch is exact in fp32."""
    rng = np.random.default_rng(seed)
    L1 = np.zeros((r, K), np.float16)
    for j in range(r):
        c = rng.choice(K, min(nnz_per_row, K), replace=False)
        L1[j, c] = rng.choice([-1, 1], size=c.size).astype(np.float16)
    L2 = rng.integers(-2, 3, size=(N, r)).astype(np.float16)
    return L1, L2


def channel_permutation(seed: int, K: int) -> np.ndarray:
    """A seeded random permutation of the K input channels (int32), standing in
    for an act-order channel order: GPTQ-R orders channels by a statistic of
    calibration data, which these synthetic layers do not have."""
    return np.random.default_rng(seed).permutation(K).astype(np.int32)


def x_outlier_channels(index: int, M: int | None = None, N: int | None = None, K: int | None = None) -> np.ndarray:
    """The activation channels ``make`` multiplies for a configuration (sorted
    int32; empty when the configuration plants none), from the same draws."""
    cfg = CONFIGS[index]
    M = cfg.Ms[0] if M is None else M
    N = cfg.N if N is None else N
    K = cfg.K if K is None else K
    if not cfg.x_outlier_channels:
        return np.zeros(0, np.int32)
    if cfg.separate_x_seeds:
        rng = np.random.default_rng(cfg.seed + M)
    else:
        rng = np.random.default_rng(cfg.seed)
        _draw_weights(rng, cfg, N, K)
    rng.standard_normal((M, K), dtype=np.float32)
    return np.sort(rng.choice(K, cfg.x_outlier_channels, replace=False)).astype(np.int32)
