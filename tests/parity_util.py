"""Shared helpers for the GPU parity tests: move seeded inputs to the GPU,
compute oracle references on the same bytes, compare per-row relative l2."""
from __future__ import annotations

import numpy as np
import torch

from oracle import harp_oracle as O

# Per-row relative l2 bounds (fp32 arithmetic in the kernels): rows stored in
# fp32 1e-5; rows stored in bf16 4e-3 (the output rounding alone contributes
# about 2^-9 / sqrt(3) ~ 1.1e-3 RMS per row).
TOL = {"f32": 1e-5, "bf16": 4e-3}

# The two-sided rotation without an fp32 workspace rounds its intermediate
# weight to bf16 between its three passes: three roundings instead of one (the
# 4e-3 bound above is for fp32 accumulation with a single output rounding).
# A bf16 rounding (8 significant bits, nearest-even) is off by at most 2^-8
# relative per element, so the bound is three of those.  On long rows the
# roundings average out well below 4e-3; rows of a few elements get close to
# the bound (15 columns: 6.5e-3, the same figure an fp64 emulation of the
# three roundings gives).
TOL_BF16_THREE_ROUNDINGS = 3 * 2.0 ** -8

BLK_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}


def to_dev(x: np.ndarray, io: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)   # exact: the values are bf16-representable
    return t.cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def oracle_blocks(schedule, d, theta, gauss, blk: str):
    exact = O.materialize_blocks(schedule, d, theta, gauss)
    return O.stored_blocks(exact, blk)


def gpu_blocks(api, schedule, d, theta, gauss, blk: str):
    th = torch.from_numpy(np.ascontiguousarray(theta, dtype=np.float64)).cuda()
    gs = torch.from_numpy(np.ascontiguousarray(gauss, dtype=np.float64)).cuda() if gauss is not None and \
        np.size(gauss) else None
    return api.harp_materialize_blocks(schedule, d, th, gs, blk)


def signs_dev(signs: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(signs, dtype=np.int8)).cuda()


def assert_rows_close(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float, label: str = ""):
    err = O.row_rel_l2(y_gpu, y_ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{label}: max per-row relative l2 {worst:.3e} > {tol:.1e} (row {int(err.argmax())})"
    return worst


def assert_groups_close(got_flat: np.ndarray, ref_blocks, schedule, tol: float, label: str = ""):
    """Per-group relative l2 of a block-layout array (dL/dB) against the
    oracle's per-stage blocks: every group's b x b block is compared on its
    own, so one group's error cannot hide under the norm of the others."""
    pos = 0
    worst = 0.0
    for t, b in enumerate(schedule):
        ref = np.asarray(ref_blocks[t], dtype=np.float64).reshape(-1, b * b)
        got = np.asarray(got_flat[pos:pos + ref.size], dtype=np.float64).reshape(-1, b * b)
        pos += ref.size
        worst = max(worst, float(O.row_rel_l2(got, ref).max()))
    assert pos == np.size(got_flat), f"{label}: {np.size(got_flat)} values for {pos} block entries"
    assert worst <= tol, f"{label}: worst per-group relative l2 {worst:.3e} > {tol:.1e}"
    return worst
