"""Named synthetic workloads (shapes, value distributions, parameter draws).

Each workload fixes a schedule, the row count, the I/O dtype and the recipe
for its seeded inputs.  ``make(name, rows=None)`` returns numpy arrays only:
rows already rounded to the I/O dtype (float32 values that are exactly
representable), int8 signs, fp64 parameters and fp64 Gaussian matrices.  The
recipes stand in for activations and weights with outlier channels and heavy
tails (the problem setting of the HARP paper); d = 4096, 5120, 8192 and the
13824 x 5120 weight are hidden / MLP widths of 7B-13B-class language models.

Master seed: 20260529 + the workload's index; streams in the order signs,
parameters, Gaussian matrices, data (see inputs.streams).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import inputs as I


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    d: int
    schedule: tuple
    rows: int
    io: str                  # "f32" or "bf16"
    sigma_skew: float = 0.0
    sigma_angle: float = 0.0
    kind: str = "apply"      # apply | rht | two_sided
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w for w in [
        Workload("sylvester64_f32", 1, 64, (2, 2, 2, 2, 2, 2), 256, "f32"),
        Workload("cayley4096_bf16", 2, 4096, (8, 8, 8, 8), 16384, "bf16", sigma_skew=0.05),
        Workload("mixed5120_bf16", 3, 5120, (8, 8, 8, 5, 2), 32768, "bf16", sigma_skew=0.05, sigma_angle=0.1),
        Workload("two_sided_13824x5120_bf16", 4, 5120, (8, 8, 8, 5, 2), 13824, "bf16", sigma_skew=0.05,
                 sigma_angle=0.05, kind="two_sided",
                 extra={"su": (8, 8, 8, 3, 3, 3), "d_out": 13824}),
        Workload("rht3_8192_bf16", 5, 8192, (8, 8, 8, 16), 65536, "bf16", kind="rht", extra={"k": 3}),
    ]
}


def round_io(x: np.ndarray, io: str) -> np.ndarray:
    """Round float32 values to the I/O dtype (bf16: nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if io == "f32":
        return x
    return I.bf16_bits_to_f32(I.f32_to_bf16_bits(x))


def _rows(w: Workload, gen: np.random.Generator, rows: int, d: int) -> np.ndarray:
    if w.index == 1:
        return I.normal_rows(gen, rows, d, outlier_coords=2, outlier_mult=30.0)
    if w.index in (2, 3):
        return I.heavy_tailed_rows(gen, rows, d, nu=3.0, outlier_frac=0.01, outlier_mult=50.0)
    if w.index == 4:
        return I.gaussian_rows(gen, rows, d, std=0.02, outlier_frac=0.005, outlier_mult=20.0)
    if w.index == 5:
        return I.adversarial_mix_rows(gen, rows, d, nu=3.0, nnz=8)
    raise ValueError(w.name)


def make(name: str, rows: int | None = None) -> dict:
    """Seeded inputs of a workload; `rows` overrides the row count (the first
    rows of a smaller draw are not the first rows of the full one)."""
    w = WORKLOADS[name]
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + w.index)
    n = w.rows if rows is None else int(rows)
    out = {"workload": w, "d": w.d, "schedule": w.schedule, "io": w.io, "rows": n}
    if w.kind == "rht":
        k = w.extra["k"]
        out["signs"] = I.rademacher(g_sign, w.d, k=k)
        out["k"] = k
    elif w.kind == "two_sided":
        su, d_out = w.extra["su"], w.extra["d_out"]
        out["su"], out["d_out"] = su, d_out
        out["signs_u"] = I.rademacher(g_sign, d_out)
        out["signs_v"] = I.rademacher(g_sign, w.d)
        out["theta_u"] = I.theta_params(g_theta, su, d_out, w.sigma_skew, w.sigma_angle)
        out["theta_v"] = I.theta_params(g_theta, w.schedule, w.d, w.sigma_skew, w.sigma_angle)
        out["gauss_u"] = I.gauss_mats(g_gauss, su)
        out["gauss_v"] = I.gauss_mats(g_gauss, w.schedule)
        n = d_out if rows is None else int(rows)
        out["rows"] = n
    else:
        out["signs"] = I.rademacher(g_sign, w.d)
        out["theta"] = I.theta_params(g_theta, w.schedule, w.d, w.sigma_skew, w.sigma_angle)
        out["gauss"] = I.gauss_mats(g_gauss, w.schedule)
    out["x"] = round_io(_rows(w, g_data, n, w.d), w.io)
    return out
