"""Seeded sweep over schedules, row counts, dtypes and entry points against the
fp64 oracle (a wider net than the per-feature tests: radices 2..16 in random
orders, every block format, with and without signs, both directions)."""
import numpy as np
import pytest
import torch

from oracle import harp_oracle as O
from structured_rotations_amd import api
from structured_rotations_amd import inputs as I
from tests.parity_util import (TOL, TOL_BF16_THREE_ROUNDINGS, assert_groups_close, assert_rows_close, from_dev, gpu_blocks, oracle_blocks,
                               signs_dev, to_dev)

pytestmark = pytest.mark.gpu

RADICES = (2, 3, 4, 5, 6, 7, 8, 9, 12, 16)

# Block gradients are sums over rows of fp32 products; per group, relative to
# the oracle's fp64 sum of the same products.
DB_TOL = 1e-5


def _cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = [((8, 8, 8), 512), ((4, 8, 4, 4), 512), ((2, 8, 8, 4), 512), ((8, 8, 4, 4, 2), 2048)]
    while len(out) < n:
        m = int(rng.integers(1, 6))
        sch = tuple(int(b) for b in rng.choice(RADICES, m))
        d = int(np.prod(sch))
        if 2 <= d <= 4096 and (sch, d) not in out:
            out.append((sch, d))
    return out


CASES = _cases(28)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_sweep(idx):
    sch, d = CASES[idx]
    rng = np.random.default_rng(1000 + idx)
    rows = int(rng.choice([1, 3, 9, 17, 33]))
    io = ["f32", "bf16"][idx % 2]
    blk = ["f32", "bf16", "i8"][idx % 3]
    use_signs = idx % 4 != 3
    print(f"\n[case] sweep {idx}: schedule {sch} d={d} rows={rows} io={io} blocks={blk} signs={use_signs}",
          flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 500 + idx)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d) if use_signs else None
    x = g_data.standard_normal((rows, d)).astype(np.float32)
    if io == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    blocks_g, scales_g = gpu_blocks(api, sch, d, theta, gauss, blk)
    blocks_o = oracle_blocks(sch, d, theta, gauss, blk)
    sg = signs_dev(signs) if use_signs else None
    s = signs.astype(float) if use_signs else None
    xd = to_dev(x, io)
    y = api.harp_apply(sch, d, blocks_g, scales_g, sg, xd)
    yd = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, xd)
    torch.cuda.synchronize()
    y_ref = O.apply(x.astype(np.float64), sch, blocks_o, s)
    assert_rows_close(from_dev(y), y_ref, TOL[io], "harp_apply")
    assert_rows_close(from_dev(yd), y_ref, TOL[io], "harp_apply_decode")
    yin = from_dev(y)
    xi = api.harp_apply_inverse(sch, d, blocks_g, scales_g, sg, y)
    xid = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, y, inverse=True)
    torch.cuda.synchronize()
    x_ref = O.apply_inverse(yin, sch, blocks_o, s)
    assert_rows_close(from_dev(xi), x_ref, TOL[io], "harp_apply_inverse")
    assert_rows_close(from_dev(xid), x_ref, TOL[io], "harp_apply_decode inverse")
    if max(sch) <= 8:
        dy = np.random.default_rng(idx).standard_normal((rows, d)).astype(np.float32)
        if io == "bf16":
            dy = torch.from_numpy(dy).to(torch.bfloat16).float().numpy()
        dx, db = api.harp_apply_vjp(sch, d, blocks_g, scales_g, sg, xd, to_dev(dy, io))
        torch.cuda.synchronize()
        rdx, rdb = O.apply_vjp(x.astype(np.float64), sch, blocks_o, s, dy.astype(np.float64))
        assert_rows_close(from_dev(dx), rdx, TOL[io], "vjp dx")
        assert_groups_close(db.cpu().numpy(), rdb, sch, DB_TOL, "vjp dB")


TWO_SIDED = [((2, 3), (5, 2)), ((4, 4), (8,)), ((3, 3, 2), (2, 5, 4)), ((8, 2), (3, 7)), ((16,), (6, 2)),
             ((5,), (4, 4, 4))]


@pytest.mark.parametrize("idx", range(len(TWO_SIDED)))
@pytest.mark.parametrize("use_ws", [False, True])
def test_sweep_two_sided(idx, use_ws):
    su, sv = TWO_SIDED[idx]
    du, dv = int(np.prod(su)), int(np.prod(sv))
    io = ["f32", "bf16"][idx % 2]
    print(f"\n[case] two-sided sweep {idx}: U {su} V {sv} io={io} workspace={use_ws} "
          f"blocks={['f32', 'bf16', 'i8'][(idx + int(use_ws)) % 3]}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 600 + idx)
    tu, tv = I.theta_params(g_theta, su, du, 0.05, 0.1), I.theta_params(g_theta, sv, dv, 0.05, 0.1)
    gu, gv = I.gauss_mats(g_gauss, su), I.gauss_mats(g_gauss, sv)
    s_u, s_v = I.rademacher(g_sign, du), I.rademacher(g_sign, dv)
    w = g_data.standard_normal((du, dv)).astype(np.float32)
    if io == "bf16":
        w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    blk = ["f32", "bf16", "i8"][(idx + int(use_ws)) % 3]
    bu, scu = gpu_blocks(api, su, du, tu, gu, blk)
    bv, scv = gpu_blocks(api, sv, dv, tv, gv, blk)
    ws = None
    if use_ws:
        ws = torch.empty(api.harp_rotate_weight_workspace(du, dv), dtype=torch.uint8, device="cuda")
    wt = api.harp_rotate_weight(su, bu, scu, signs_dev(s_u), sv, bv, scv, signs_dev(s_v), to_dev(w, io),
                                workspace=ws, fp32_intermediates=use_ws)
    torch.cuda.synchronize()
    obu, obv = oracle_blocks(su, du, tu, gu, blk), oracle_blocks(sv, dv, tv, gv, blk)
    ref = O.rotate_weight(w.astype(np.float64), su, obu, s_u.astype(float), sv, obv, s_v.astype(float))
    # every row of the rotated weight on its own; bf16 without a workspace
    # rounds between the passes (three roundings)
    tol = TOL_BF16_THREE_ROUNDINGS if (io == "bf16" and not use_ws) else TOL[io]
    assert_rows_close(from_dev(wt), ref, tol, "two-sided sweep")


RHT = [((2, 2, 2), 8, 1), ((4, 16), 64, 2), ((8, 8, 8), 512, 3), ((16, 2, 8), 256, 5)]


@pytest.mark.parametrize("idx", range(len(RHT)))
@pytest.mark.parametrize("inverse", [False, True])
def test_sweep_rht(idx, inverse):
    sch, d, k = RHT[idx]
    io = ["f32", "bf16"][idx % 2]
    print(f"\n[case] rht sweep {idx}: {sch} k={k} io={io} inverse={inverse}", flush=True)
    g_sign, _, _, g_data = I.streams(I.BASE_SEED + 700 + idx)
    signs = I.rademacher(g_sign, d, k=k)
    x = g_data.standard_normal((13, d)).astype(np.float32)
    if io == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    y = api.rht_compose(sch, d, signs_dev(signs), to_dev(x, io), inverse=inverse)
    torch.cuda.synchronize()
    ref = O.rht_compose(x.astype(np.float64), np.asarray(signs, dtype=float).reshape(k, d), inverse=inverse)
    assert_rows_close(from_dev(y), ref, TOL[io], "rht_compose")


def _large_cases(n, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        m = int(rng.integers(2, 7))
        sch = tuple(int(b) for b in rng.choice(RADICES, m))
        d = int(np.prod(sch))
        if 4096 < d <= 16384 and (sch, d) not in out:
            out.append((sch, d))
    return out


LARGE = _large_cases(8)


@pytest.mark.parametrize("idx", range(len(LARGE)))
def test_sweep_large_d(idx):
    # d from 4097 to 16384 in random mixed-radix orders; row counts on both
    # sides of the decode entry point's hand-over to the row kernels (128)
    sch, d = LARGE[idx]
    rows = [1, 7, 64, 129, 300][idx % 5]
    io = ["f32", "bf16"][idx % 2]
    blk = ["f32", "bf16", "i8"][idx % 3]
    print(f"\n[case] large-d sweep {idx}: schedule {sch} d={d} rows={rows} io={io} blocks={blk}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 900 + idx)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    x = g_data.standard_normal((rows, d)).astype(np.float32)
    if io == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    blocks_g, scales_g = gpu_blocks(api, sch, d, theta, gauss, blk)
    blocks_o = oracle_blocks(sch, d, theta, gauss, blk)
    sg, s = signs_dev(signs), signs.astype(float)
    xd = to_dev(x, io)
    y = api.harp_apply(sch, d, blocks_g, scales_g, sg, xd)
    yd = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, xd)
    torch.cuda.synchronize()
    y_ref = O.apply(x.astype(np.float64), sch, blocks_o, s)
    assert_rows_close(from_dev(y), y_ref, TOL[io], "harp_apply")
    assert_rows_close(from_dev(yd), y_ref, TOL[io], "harp_apply_decode")
    yin = from_dev(y)
    xi = api.harp_apply_inverse(sch, d, blocks_g, scales_g, sg, y)
    torch.cuda.synchronize()
    assert_rows_close(from_dev(xi), O.apply_inverse(yin, sch, blocks_o, s), TOL[io], "harp_apply_inverse")
    if max(sch) <= 8:
        dy = np.random.default_rng(idx).standard_normal((rows, d)).astype(np.float32)
        if io == "bf16":
            dy = torch.from_numpy(dy).to(torch.bfloat16).float().numpy()
        dx, db = api.harp_apply_vjp(sch, d, blocks_g, scales_g, sg, xd, to_dev(dy, io))
        torch.cuda.synchronize()
        rdx, rdb = O.apply_vjp(x.astype(np.float64), sch, blocks_o, s, dy.astype(np.float64))
        assert_rows_close(from_dev(dx), rdx, TOL[io], "vjp dx")
        assert_groups_close(db.cpu().numpy(), rdb, sch, DB_TOL, "vjp dB")
