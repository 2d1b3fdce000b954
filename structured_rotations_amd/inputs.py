"""Seeded synthetic inputs shared by the tests, the bench and the oracle legs.

This module draws random numbers and converts them to the storage formats the
library reads (bfloat16 bit patterns, fp32, int8).  It holds none of the
transform's arithmetic: no base mixers, no Givens or Cayley maps, no stages.
Random numbers the method itself needs (the Gaussian matrices behind the QR
base mixer, the learnable parameters, the sign vectors) are drawn here and
handed to both sides as inputs.

Every draw goes through numpy's PCG64 seeded by ``SeedSequence(seed)``; the
spawned child streams are used in a fixed order: signs, parameters, Gaussian
base-mixer matrices, data.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20260529


def streams(seed: int, n: int = 4) -> list[np.random.Generator]:
    """Independent child generators: [signs, theta, gauss, data, ...]."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def rademacher(gen: np.random.Generator, d: int, k: int | None = None) -> np.ndarray:
    """Random +-1 signs as int8, shape (d,) or (k, d)."""
    shape = (d,) if k is None else (k, d)
    return np.where(gen.integers(0, 2, size=shape) == 1, 1, -1).astype(np.int8)


def is_pow2(b: int) -> bool:
    return b >= 1 and (b & (b - 1)) == 0


def theta_params(gen: np.random.Generator, schedule, d: int,
                 sigma_skew: float, sigma_angle: float) -> np.ndarray:
    """Learnable parameters, concatenated over stages: one normal angle per
    group for radix 2 (std sigma_angle), b(b-1)/2 normal skew entries per group
    otherwise (std sigma_skew).  sigma 0 gives the all-zero initialisation."""
    parts = []
    for b in schedule:
        ngroups = d // b
        if b == 2:
            parts.append(gen.standard_normal(ngroups) * sigma_angle)
        else:
            parts.append(gen.standard_normal(ngroups * (b * (b - 1) // 2)) * sigma_skew)
    return np.concatenate(parts) if parts else np.zeros(0)


def gauss_mats(gen: np.random.Generator, schedule) -> np.ndarray:
    """One standard-normal b x b matrix per distinct non-power-of-two radix,
    replicated for every stage with that radix (concatenated in stage order)."""
    per_radix: dict[int, np.ndarray] = {}
    parts = []
    for b in schedule:
        if is_pow2(b):
            continue
        if b not in per_radix:
            per_radix[b] = gen.standard_normal((b, b))
        parts.append(per_radix[b].ravel())
    return np.concatenate(parts) if parts else np.zeros(0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(gen: np.random.Generator, d: int, frac: float) -> np.ndarray:
    """floor(frac * d) distinct channel indices, drawn without replacement."""
    n = int(np.floor(frac * d))
    return np.sort(gen.choice(d, size=n, replace=False)) if n > 0 else np.zeros(0, dtype=np.int64)


def heavy_tailed_rows(gen: np.random.Generator, rows: int, d: int, nu: float,
                      outlier_frac: float, outlier_mult: float,
                      chunk: int = 4096) -> np.ndarray:
    """Student-t rows (unit scale) with a fixed set of outlier channels scaled
    by outlier_mult in every row; float32 output, generated in row chunks."""
    ch = outlier_channels(gen, d, outlier_frac)
    out = np.empty((rows, d), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        blk = gen.standard_t(nu, size=(r1 - r0, d))
        if ch.size:
            blk[:, ch] *= outlier_mult
        out[r0:r1] = blk
    return out


def gaussian_rows(gen: np.random.Generator, rows: int, d: int, std: float,
                  outlier_frac: float, outlier_mult: float, n_outlier_fixed: int | None = None,
                  chunk: int = 4096) -> np.ndarray:
    """N(0, std^2) rows with outlier channels (columns) scaled by outlier_mult."""
    if n_outlier_fixed is not None:
        ch = np.sort(gen.choice(d, size=n_outlier_fixed, replace=False))
    else:
        ch = outlier_channels(gen, d, outlier_frac)
    out = np.empty((rows, d), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        blk = gen.standard_normal((r1 - r0, d)) * std
        if ch.size:
            blk[:, ch] *= outlier_mult
        out[r0:r1] = blk
    return out


def adversarial_mix_rows(gen: np.random.Generator, rows: int, d: int, nu: float,
                         nnz: int = 8, chunk: int = 4096) -> np.ndarray:
    """A quarter one-hot rows (1.0 at a random index), a quarter rows with
    exactly nnz standard-normal entries at distinct random positions, half
    Student-t rows; row order shuffled."""
    n_onehot = rows // 4
    n_sparse = rows // 4
    kinds = np.concatenate([np.zeros(n_onehot, np.int8), np.ones(n_sparse, np.int8),
                            np.full(rows - n_onehot - n_sparse, 2, np.int8)])
    gen.shuffle(kinds)
    out = np.zeros((rows, d), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        k = kinds[r0:r1]
        blk = np.zeros((r1 - r0, d), dtype=np.float64)
        dense = np.nonzero(k == 2)[0]
        if dense.size:
            blk[dense] = gen.standard_t(nu, size=(dense.size, d))
        for i in np.nonzero(k == 0)[0]:
            blk[i, gen.integers(0, d)] = 1.0
        for i in np.nonzero(k == 1)[0]:
            pos = gen.choice(d, size=nnz, replace=False)
            blk[i, pos] = gen.standard_normal(nnz)
        out[r0:r1] = blk
    return out


def normal_rows(gen: np.random.Generator, rows: int, d: int, outlier_coords: int = 0,
                outlier_mult: float = 1.0) -> np.ndarray:
    """N(0,1) rows with a fixed set of outlier coordinates in every row."""
    ch = np.sort(gen.choice(d, size=outlier_coords, replace=False)) if outlier_coords else None
    x = gen.standard_normal((rows, d))
    if ch is not None:
        x[:, ch] *= outlier_mult
    return x.astype(np.float32)
