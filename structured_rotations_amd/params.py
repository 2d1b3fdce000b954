"""Saving and loading a fitted processor: the schedule, Θ (or its int8 codes
and per-stage scales), the Gaussian base mixers of the non-power-of-two
stages, the Rademacher signs and the seeds they were drawn from.

These are the only state of the path (HARP technical summary §2.2: the
blocks are materialised from Θ and the fixed base mixers; §4: Θ stored as
int8).  The file is a plain .npz; loading never unpickles (allow_pickle is
off), and the arrays are checked against the schedule's sizes.
"""
from __future__ import annotations

import numpy as np

_FORMAT = 1


def _theta_count(schedule, d: int) -> int:
    # one angle per group for radix 2, b(b-1)/2 skew entries otherwise
    return sum((d // b) * (1 if b == 2 else b * (b - 1) // 2) for b in schedule)


def _gauss_count(schedule) -> int:
    return sum(b * b for b in schedule if b & (b - 1))


def save_params(path, schedule, d: int, signs, theta=None, gauss=None, theta_codes=None, theta_scales=None,
                seeds=None) -> None:
    """Writes one processor to `path` (.npz).  Give Θ as fp64 `theta`, or as
    int8 `theta_codes` with one fp32 scale per stage (`theta_scales`), or both."""
    schedule = np.asarray(schedule, dtype=np.int32)
    if int(np.prod(schedule)) != int(d):
        raise ValueError("product of the schedule != d")
    if theta is None and theta_codes is None:
        raise ValueError("give theta or theta_codes")
    if (theta_codes is None) != (theta_scales is None):
        raise ValueError("theta_codes and theta_scales go together")
    arrays = {"format": np.array(_FORMAT, dtype=np.int32), "schedule": schedule,
              "d": np.array(int(d), dtype=np.int64), "signs": np.ascontiguousarray(signs, dtype=np.int8)}
    if theta is not None:
        arrays["theta"] = np.ascontiguousarray(theta, dtype=np.float64)
    if theta_codes is not None:
        arrays["theta_codes"] = np.ascontiguousarray(theta_codes, dtype=np.int8)
        arrays["theta_scales"] = np.ascontiguousarray(theta_scales, dtype=np.float32)
    arrays["gauss"] = np.ascontiguousarray(gauss if gauss is not None else np.zeros(0), dtype=np.float64)
    if seeds is not None:
        arrays["seeds"] = np.asarray(seeds, dtype=np.int64)
    _check(arrays)
    np.savez(path, **arrays)


def load_params(path) -> dict:
    """Reads a file written by save_params; returns a dict with the same keys
    (schedule as a tuple, d as an int)."""
    with np.load(path, allow_pickle=False) as f:
        arrays = {k: f[k] for k in f.files}
    if int(arrays.get("format", -1)) != _FORMAT:
        raise ValueError("not a parameter file of this format")
    _check(arrays)
    out = dict(arrays)
    out["schedule"] = tuple(int(b) for b in arrays["schedule"])
    out["d"] = int(arrays["d"])
    del out["format"]
    return out


def _check(a: dict) -> None:
    sch = [int(b) for b in a["schedule"]]
    d = int(a["d"])
    if any(b < 2 or b > 16 for b in sch) or int(np.prod(sch)) != d:
        raise ValueError("invalid schedule")
    if a["signs"].ndim != 1 or a["signs"].size != d or not np.all(np.abs(a["signs"]) == 1):
        raise ValueError("signs must be d entries of +-1")
    n = _theta_count(sch, d)
    if "theta" in a and a["theta"].size != n:
        raise ValueError(f"theta has {a['theta'].size} entries, the schedule needs {n}")
    if "theta_codes" in a:
        if a["theta_codes"].size != n or a["theta_scales"].size != len(sch):
            raise ValueError("theta_codes / theta_scales sizes do not match the schedule")
    if a["gauss"].size != _gauss_count(sch):
        raise ValueError(f"gauss has {a['gauss'].size} entries, the schedule needs {_gauss_count(sch)}")
