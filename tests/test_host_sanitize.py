"""The host C++ of the boundary (schedule planner and row-argument validation,
structured_rotations_amd/csrc/plan.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/host/plan_check.cpp is built with g++ (no HIP) and run: randomized
schedules, valid and invalid, and randomized row arguments including extreme
sizes, leading dimensions and pointers; any out-of-bounds access, signed
overflow or other undefined behaviour aborts it.  The plan's per-stage
offsets are then compared with the oracle's parameter counts (HARP technical
summary §2.1-§2.2: one b x b block per group, b(b-1)/2 skew parameters per
group or one angle for b = 2, one Gaussian base mixer per non-power-of-two
stage).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import harp_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_rotations_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("host") / "plan_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(ROOT, "tests", "host", "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return str(out)


def test_randomized_planner_and_row_checks(plan_check):
    r = subprocess.run([plan_check], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def _plan(plan_check, sch, d):
    r = subprocess.run([plan_check, "print", str(d)] + [str(b) for b in sch], capture_output=True, text=True,
                       timeout=60, env=ENV)
    assert r.returncode == 0, r.stderr
    return dict(line.split("=", 1) for line in r.stdout.split("\n") if "=" in line)


@pytest.mark.parametrize("sch", [(2,), (8, 8, 8, 8), (8, 8, 8, 5, 2), (8, 8, 8, 3, 3, 3), (3, 7, 16, 2),
                                 (16, 16, 16), (6, 5, 2)])
def test_plan_matches_oracle_counts(plan_check, sch):
    d = int(np.prod(sch))
    kv = _plan(plan_check, sch, d)
    ints = lambda k: [int(v) for v in kv[k].split(",")]
    theta = O.theta_counts(sch, d)
    assert int(kv["n_theta"]) == sum(theta)
    assert ints("theta_off") == [int(v) for v in np.concatenate([[0], np.cumsum(theta)[:-1]])]
    # block layout: the oracle's materialised blocks, stage by stage
    rng = np.random.default_rng(3)
    gs = O.gauss_stage_list(sch)
    gauss = rng.standard_normal(sum(sch[t] ** 2 for t in gs)) if gs else None
    blocks = O.materialize_blocks(sch, d, rng.standard_normal(sum(theta)) * 0.1, gauss)
    sizes = [blocks[t].size for t in range(len(sch))]
    assert int(kv["n_blk"]) == sum(sizes)
    assert ints("blk_off") == [int(v) for v in np.concatenate([[0], np.cumsum(sizes)[:-1]])]
    assert ints("grp_off") == [int(v) for v in np.concatenate([[0], np.cumsum([d // b for b in sch])[:-1]])]
    # Gaussian base mixers: only the non-power-of-two stages, b*b each, in stage order
    goff, pos = [], 0
    for t, b in enumerate(sch):
        goff.append(pos if t in gs else -1)
        pos += b * b if t in gs else 0
    assert ints("gauss_off") == goff and int(kv["n_gauss"]) == pos
    # digit strides: stage t mixes the digit of stride prod_{u>t} b_u
    assert ints("stride") == [int(np.prod(sch[t + 1:])) for t in range(len(sch))]


def test_plan_rejections(plan_check):
    assert "error" in _plan(plan_check, (3, 3), 10)      # product != d
    assert "error" in _plan(plan_check, (17, 2), 34)     # radix above 16
    assert "error" in _plan(plan_check, (1, 8), 8)       # radix below 2
