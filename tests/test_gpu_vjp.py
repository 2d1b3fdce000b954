"""Parity of the reverse-mode kernels (through the C ABI) with the fp64 oracle.

dx is compared per row as the forward path is (relative l2 <= 1e-5 for fp32
rows, <= 4e-3 for bf16 rows, the latter set by the output rounding).  The
block gradients are fp32 sums over rows of products of fp32 intermediates;
they are compared per group: relative l2 <= 1e-5 (each product is exact to
2^-24 relative, and the sums run over at most a few hundred terms per chunk
plus one add per chunk).  The parameter gradient runs in fp64 from fp32 block
gradients and is compared against the oracle fed the same fp32 values.
"""
import numpy as np
import pytest
import torch

from oracle import harp_oracle as O
from structured_rotations_amd import api
from structured_rotations_amd import inputs as I
from structured_rotations_amd import workloads as W
from structured_rotations_amd._lib import HarpError
from tests.parity_util import (TOL, assert_groups_close, assert_rows_close, from_dev, gpu_blocks, oracle_blocks, signs_dev, to_dev)

pytestmark = pytest.mark.gpu

DB_TOL = 1e-5


def _dy(rows, d, io, seed):
    g = np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32)
    if io == "bf16":
        g = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
    return g


@pytest.mark.parametrize("name", ["sylvester64_f32", "cayley4096_bf16", "mixed5120_bf16"])
@pytest.mark.parametrize("blk", ["f32", "bf16", "i8"])
def test_vjp_matches_oracle(name, blk):
    rows = 37
    print(f"\n[case] vjp {name} blk={blk} rows={rows}", flush=True)
    w = W.make(name, rows)
    sch, d, io = w["schedule"], w["d"], w["io"]
    blocks_g, scales_g = gpu_blocks(api, sch, d, w["theta"], w["gauss"], blk)
    sg = signs_dev(w["signs"])
    dy = _dy(rows, d, io, 5)
    dx, db = api.harp_apply_vjp(sch, d, blocks_g, scales_g, sg, to_dev(w["x"], io), to_dev(dy, io))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], blk)
    rdx, rdb = O.apply_vjp(w["x"].astype(np.float64), sch, blocks_o, w["signs"].astype(float), dy.astype(np.float64))
    assert_rows_close(from_dev(dx), rdx, TOL[io], f"{name}/{blk} dx")
    assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, f"{name}/{blk} dB")


@pytest.mark.parametrize("sch,d", [((8, 8, 8, 3, 3, 3), 13824), ((2, 5, 4), 40), ((7,), 7), ((3, 2, 6), 36)])
def test_vjp_other_schedules(sch, d):
    print(f"\n[case] vjp schedule {sch}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 200 + d)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    rows = 11
    x = g_data.standard_normal((rows, d)).astype(np.float32)
    dy = _dy(rows, d, "f32", 6)
    blocks_g, _ = gpu_blocks(api, sch, d, theta, gauss, "f32")
    dx, db = api.harp_apply_vjp(sch, d, blocks_g, None, signs_dev(signs), to_dev(x, "f32"), to_dev(dy, "f32"))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, theta, gauss, "f32")
    rdx, rdb = O.apply_vjp(x.astype(np.float64), sch, blocks_o, signs.astype(float), dy.astype(np.float64))
    assert_rows_close(from_dev(dx), rdx, TOL["f32"], f"{sch} dx")
    assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, f"{sch} dB")


@pytest.mark.parametrize("name", ["cayley4096_bf16", "mixed5120_bf16"])
def test_theta_vjp_matches_oracle(name):
    print(f"\n[case] theta vjp {name}", flush=True)
    w = W.make(name, 1)
    sch, d = w["schedule"], w["d"]
    rng = np.random.default_rng(21)
    dblocks = rng.standard_normal(api.harp_block_count(sch, d)).astype(np.float32)
    th = torch.from_numpy(w["theta"]).cuda()
    gs = torch.from_numpy(w["gauss"]).cuda() if w["gauss"].size else None
    dt = api.harp_theta_vjp(sch, d, th, gs, torch.from_numpy(dblocks).cuda())
    torch.cuda.synchronize()
    pos, split = 0, []
    for b in sch:
        split.append(dblocks[pos:pos + d * b].astype(np.float64).reshape(d // b, b, b))
        pos += d * b
    ref = O.theta_vjp(sch, d, w["theta"], w["gauss"], split)
    got = dt.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_vjp_full_chain_to_theta_at_calibration_size():
    # A 4096-row batch (one weight's rows) through the GPU chain
    # x, dy -> dB -> dtheta against the oracle chain in fp64.
    rows = 4096
    w = W.make("mixed5120_bf16", rows)
    print(f"\n[case] vjp full chain mixed5120 rows={rows}", flush=True)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "f32")
    dy = _dy(rows, d, "bf16", 7)
    _, db = api.harp_apply_vjp(sch, d, blocks_g, None, signs_dev(w["signs"]), to_dev(w["x"], "bf16"),
                               to_dev(dy, "bf16"), want_dx=False)
    th = torch.from_numpy(w["theta"]).cuda()
    gs = torch.from_numpy(w["gauss"]).cuda()
    dt = api.harp_theta_vjp(sch, d, th, gs, db)
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], "f32")
    _, rdb = O.apply_vjp(w["x"].astype(np.float64), sch, blocks_o, w["signs"].astype(float), dy.astype(np.float64))
    assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, "full dB")
    rdt = O.theta_vjp(sch, d, w["theta"], w["gauss"], rdb)
    got = dt.cpu().numpy()
    pos = 0
    for n_t in O.theta_counts(sch, d):
        g, r = got[pos:pos + n_t], rdt[pos:pos + n_t]
        assert np.linalg.norm(g - r) <= DB_TOL * np.linalg.norm(r), "dtheta per stage"
        pos += n_t


def test_vjp_errors_and_no_dx():
    w = W.make("cayley4096_bf16", 3)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "f32")
    sg = signs_dev(w["signs"])
    x = to_dev(w["x"], "bf16")
    need = api.harp_apply_vjp_workspace(sch, d, 3)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dx, db = api.harp_apply_vjp(sch, d, blocks_g, None, sg, x, x, want_dx=False, workspace=ws)
    torch.cuda.synchronize()
    assert dx is None and torch.isfinite(db).all()
    with pytest.raises(HarpError):
        api.harp_apply_vjp(sch, d, blocks_g, None, sg, x, x, workspace=ws[:need - 4])
    assert api.harp_apply_vjp_workspace((16, 16), 256, 3) == -1


def test_vjp_without_signs_and_one_row():
    w = W.make("cayley4096_bf16", 1)
    sch, d = w["schedule"], w["d"]
    print("\n[case] vjp cayley4096 rows=1 no signs", flush=True)
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "f32")
    dy = _dy(1, d, "f32", 8)
    dx, db = api.harp_apply_vjp(sch, d, blocks_g, None, None, to_dev(w["x"], "f32"), to_dev(dy, "f32"))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], "f32")
    rdx, rdb = O.apply_vjp(w["x"].astype(np.float64), sch, blocks_o, None, dy.astype(np.float64))
    assert_rows_close(from_dev(dx), rdx, TOL["f32"], "dx")
    assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, "dB")


@pytest.mark.parametrize("sch,d", [((8, 8, 8, 8), 4096), ((4, 8, 4), 128)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("pad", [0, 1, 8])
def test_vjp_strided_rows(sch, d, io, pad):
    """Row strides that keep or break the 16-byte alignment of the stride-1
    stage's contiguous group accesses (dx and dB both checked); rows span
    more than one row chunk per workgroup."""
    print(f"\n[case] vjp strided {sch} io={io} pad={pad}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 300 + d + pad)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    rows = 300
    x = g_data.standard_normal((rows, d)).astype(np.float32)
    dy = _dy(rows, d, io, 9)
    if io == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    tdt = torch.bfloat16 if io == "bf16" else torch.float32

    def wide(a):
        t = torch.zeros((rows, d + pad), dtype=tdt, device="cuda")
        t[:, :d] = torch.from_numpy(a).to(tdt).cuda()
        return t[:, :d]

    xd, dyd = wide(x), wide(dy)
    dx = torch.full((rows, d + pad), 7.0, dtype=tdt, device="cuda")[:, :d]
    blocks_g, _ = gpu_blocks(api, sch, d, theta, gauss, "f32")
    _, db = api.harp_apply_vjp(sch, d, blocks_g, None, signs_dev(signs), xd, dyd, dx=dx)
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, theta, gauss, "f32")
    rdx, rdb = O.apply_vjp(x.astype(np.float64), sch, blocks_o, signs.astype(float), dy.astype(np.float64))
    assert_rows_close(dx.float().cpu().numpy(), rdx, TOL[io], f"{sch}/{io}/pad{pad} dx")
    assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, f"{sch}/{io}/pad{pad} dB")
    if pad:
        base = dx.as_strided((rows, pad), (d + pad, 1), d)   # the pad columns beside each row
        assert bool((base.float() == 7.0).all()), "dx written outside its rows"


@pytest.mark.parametrize("sch,d", [((8, 8), 64), ((3, 8, 8), 192), ((2, 2, 8, 8), 256), ((5, 2), 10),
                                   ((3, 5, 2), 30), ((7, 5, 2), 70), ((3, 3), 9), ((2, 3, 3), 18),
                                   ((8, 8, 3, 3), 576)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("blk", ["f32", "i8"])
def test_vjp_fused_last_pair(sch, d, io, blk):
    """Schedules ending in a compiled-in pair of stages ((8, 8), (5, 2),
    (3, 3)) take the fused backward launch for that pair (with m = 2 it reads
    x and writes dx itself, signs on both sides); units that leave lanes of a
    wave idle, sets of units past the last one, and row counts that leave
    partial row groups and empty chunks."""
    print(f"\n[case] vjp fused pair {sch} io={io} blk={blk}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 400 + d)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    for rows in (1, 13, 517):
        x = g_data.standard_normal((rows, d)).astype(np.float32)
        if io == "bf16":
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        dy = _dy(rows, d, io, 10 + rows)
        blocks_g, scales_g = gpu_blocks(api, sch, d, theta, gauss, blk)
        dx, db = api.harp_apply_vjp(sch, d, blocks_g, scales_g, signs_dev(signs), to_dev(x, io), to_dev(dy, io))
        torch.cuda.synchronize()
        blocks_o = oracle_blocks(sch, d, theta, gauss, blk)
        rdx, rdb = O.apply_vjp(x.astype(np.float64), sch, blocks_o, signs.astype(float), dy.astype(np.float64))
        assert_rows_close(from_dev(dx), rdx, TOL[io], f"{sch}/{io}/{blk}/{rows} dx")
        assert_groups_close(db.cpu().numpy().astype(np.float64), rdb, sch, DB_TOL, f"{sch}/{io}/{blk}/{rows} dB")
