"""Parity of the small-batch (decode) apply with the fp64 oracle, through the C ABI.

Same bounds as the row path: per-row relative l2 <= 1e-5 for fp32 rows and
<= 4e-3 for bf16 rows, against the oracle on the same input bytes and the
same stored block values.  Row counts span the per-token regime (1 row), a
ragged row block, several row blocks, and the most rows the entry point takes.
"""
import numpy as np
import pytest
import torch

from oracle import harp_oracle as O
from structured_rotations_amd import api
from structured_rotations_amd import inputs as I
from structured_rotations_amd import workloads as W
from structured_rotations_amd._lib import HarpError
from tests.parity_util import (TOL, assert_rows_close, from_dev, gpu_blocks, oracle_blocks, signs_dev, to_dev)

pytestmark = pytest.mark.gpu


def _case(name, rows):
    print(f"\n[case] decode {name} rows={rows}", flush=True)
    return W.make(name, rows)


@pytest.mark.parametrize("name", ["sylvester64_f32", "cayley4096_bf16", "mixed5120_bf16"])
@pytest.mark.parametrize("blk", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("rows", [1, 5, 64])
def test_decode_matches_oracle(name, blk, rows):
    w = _case(name, rows)
    sch, d, io = w["schedule"], w["d"], w["io"]
    blocks_g, scales_g = gpu_blocks(api, sch, d, w["theta"], w["gauss"], blk)
    sg = signs_dev(w["signs"])
    y = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, to_dev(w["x"], io))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], blk)
    s = w["signs"].astype(float)
    assert_rows_close(from_dev(y), O.apply(w["x"].astype(np.float64), sch, blocks_o, s), TOL[io],
                      f"{name}/{blk}/{rows} forward")
    yin = from_dev(y)
    xr = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, y, inverse=True)
    torch.cuda.synchronize()
    assert_rows_close(from_dev(xr), O.apply_inverse(yin, sch, blocks_o, s), TOL[io], f"{name}/{blk}/{rows} inverse")


OTHER = [((8, 8, 8, 3, 3, 3), 13824), ((3, 7, 16, 2), 672), ((16, 16, 16), 4096), ((2, 5, 4), 40),
         ((4, 4, 4, 4, 4), 1024), ((8, 8, 8, 16), 8192)]


@pytest.mark.parametrize("sch,d", OTHER)
@pytest.mark.parametrize("blk", ["f32", "i8"])
def test_decode_other_schedules(sch, d, blk):
    print(f"\n[case] decode schedule {sch} blk={blk}", flush=True)
    g_sign, g_theta, g_gauss, g_data = I.streams(I.BASE_SEED + 100 + d)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    rows = 9
    x = g_data.standard_normal((rows, d)).astype(np.float32)
    blocks_g, scales_g = gpu_blocks(api, sch, d, theta, gauss, blk)
    blocks_o = oracle_blocks(sch, d, theta, gauss, blk)
    sg = signs_dev(signs)
    xd = to_dev(x, "f32")
    y = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, xd)
    xr = api.harp_apply_decode(sch, d, blocks_g, scales_g, sg, y, inverse=True)
    torch.cuda.synchronize()
    s = signs.astype(float)
    y_ref = O.apply(x.astype(np.float64), sch, blocks_o, s)
    assert_rows_close(from_dev(y), y_ref, TOL["f32"], f"{sch} forward")
    assert_rows_close(from_dev(xr), O.apply_inverse(from_dev(y), sch, blocks_o, s), TOL["f32"], f"{sch} inverse")


def test_decode_max_rows_hands_over_to_row_kernels():
    # 1024 rows: above 128 rows the call runs the throughput row kernels.
    w = _case("cayley4096_bf16", 1024)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "bf16")
    y = api.harp_apply_decode(sch, d, blocks_g, None, signs_dev(w["signs"]), to_dev(w["x"], "bf16"))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], "bf16")
    y_ref = O.apply(w["x"].astype(np.float64), sch, blocks_o, w["signs"].astype(float))
    assert_rows_close(from_dev(y), y_ref, TOL["bf16"], "1024 rows")


def test_decode_sub_problem_chunks():
    # 128 rows of a (4,4,4,4,4) schedule: no compile-time kernel for its runs,
    # and the generic kernel puts two sub-problems in each workgroup.
    sch, d = (4, 4, 4, 4, 4), 1024
    print(f"\n[case] decode {sch} rows=128", flush=True)
    g_sign, g_theta, _, g_data = I.streams(I.BASE_SEED + 400)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    signs = I.rademacher(g_sign, d)
    x = g_data.standard_normal((128, d)).astype(np.float32)
    blocks_g, _ = gpu_blocks(api, sch, d, theta, None, "f32")
    y = api.harp_apply_decode(sch, d, blocks_g, None, signs_dev(signs), to_dev(x, "f32"))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, theta, None, "f32")
    y_ref = O.apply(x.astype(np.float64), sch, blocks_o, signs.astype(float))
    assert_rows_close(from_dev(y), y_ref, TOL["f32"], "128 rows, two sub-problems per workgroup")


def test_decode_in_place_strided_workspace_and_errors():
    w = _case("mixed5120_bf16", 7)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "f32")
    sg = signs_dev(w["signs"])
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], "f32")
    y_ref = O.apply(w["x"].astype(np.float64), sch, blocks_o, w["signs"].astype(float))
    need = api.harp_apply_decode_workspace(sch, d, "f32", 7)
    assert need == 7 * d * 4
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    # strided rows, output padding untouched
    big = torch.zeros(7, d + 24, dtype=torch.bfloat16, device="cuda")
    big[:, :d] = to_dev(w["x"], "bf16")
    out = torch.full((7, d + 40), 7.0, dtype=torch.bfloat16, device="cuda")
    api.harp_apply_decode(sch, d, blocks_g, None, sg, big[:, :d], out[:, :d], workspace=ws)
    # in place
    xd = to_dev(w["x"], "bf16")
    api.harp_apply_decode(sch, d, blocks_g, None, sg, xd, xd, workspace=ws)
    torch.cuda.synchronize()
    assert_rows_close(from_dev(out[:, :d]), y_ref, TOL["bf16"], "strided")
    assert torch.all(out[:, d:] == 7.0)
    assert_rows_close(from_dev(xd), y_ref, TOL["bf16"], "in place")
    with pytest.raises(HarpError):
        api.harp_apply_decode(sch, d, blocks_g, None, sg, xd, workspace=ws[:need - 4])
    with pytest.raises(HarpError):
        api.harp_apply_decode(sch, d, blocks_g, None, sg,
                              torch.zeros(1025, d, dtype=torch.bfloat16, device="cuda"))
    empty = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    api.harp_apply_decode(sch, d, blocks_g, None, sg, empty, empty.clone())


def test_decode_single_launch_needs_no_workspace():
    w = _case("sylvester64_f32", 3)
    assert api.harp_apply_decode_workspace(w["schedule"], w["d"], "f32", 3) == 0


def test_decode_graph_replays_match_eager():
    # The decode calls captured in a HIP graph (no memset nodes: the kernels
    # write every output element) and replayed several times, with eager work
    # and synchronisation between replays; each replay equals the eager result.
    w = _case("cayley4096_bf16", 4)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "bf16")
    sg = signs_dev(w["signs"])
    x = to_dev(w["x"], "bf16")
    ws = torch.empty(api.harp_apply_decode_workspace(sch, d, "bf16", 4), dtype=torch.uint8, device="cuda")
    y_eager = api.harp_apply_decode(sch, d, blocks_g, None, sg, x, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.harp_apply_decode(sch, d, blocks_g, None, sg, x, y, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)


def test_decode_unaligned_blocks_and_largest_row():
    # Blocks 4 bytes off a 16-byte boundary take the generic kernel; d = 32768
    # (the largest row) splits into runs of 64 and 512.
    sch, d = (8, 8, 8, 8, 8), 32768
    print(f"\n[case] decode {sch} unaligned blocks", flush=True)
    g_sign, g_theta, _, g_data = I.streams(I.BASE_SEED + 300)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    signs = I.rademacher(g_sign, d)
    x = g_data.standard_normal((3, d)).astype(np.float32)
    blocks_g, _ = gpu_blocks(api, sch, d, theta, None, "f32")
    shifted = torch.empty(blocks_g.numel() + 1, dtype=torch.float32, device="cuda")[1:]
    shifted.copy_(blocks_g)
    assert shifted.data_ptr() % 16 != 0
    sg = signs_dev(signs)
    y_al = api.harp_apply_decode(sch, d, blocks_g, None, sg, to_dev(x, "f32"))
    y_un = api.harp_apply_decode(sch, d, shifted, None, sg, to_dev(x, "f32"))
    y_ap = api.harp_apply(sch, d, blocks_g, None, sg, to_dev(x, "f32"))
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, theta, None, "f32")
    y_ref = O.apply(x.astype(np.float64), sch, blocks_o, signs.astype(float))
    assert_rows_close(from_dev(y_al), y_ref, TOL["f32"], "aligned")
    assert_rows_close(from_dev(y_un), y_ref, TOL["f32"], "unaligned")
    assert_rows_close(from_dev(y_ap), y_ref, TOL["f32"], "harp_apply at d = 32768")


@pytest.mark.parametrize("inverse", [False, True])
def test_decode_without_signs(inverse):
    # signs = NULL is D_s = I on both entry points.
    w = _case("mixed5120_bf16", 3)
    sch, d = w["schedule"], w["d"]
    blocks_g, _ = gpu_blocks(api, sch, d, w["theta"], w["gauss"], "f32")
    x = to_dev(w["x"], "f32")
    y = api.harp_apply_decode(sch, d, blocks_g, None, None, x, inverse=inverse)
    torch.cuda.synchronize()
    blocks_o = oracle_blocks(sch, d, w["theta"], w["gauss"], "f32")
    fn = O.apply_inverse if inverse else O.apply
    assert_rows_close(from_dev(y), fn(w["x"].astype(np.float64), sch, blocks_o, None), TOL["f32"], "no signs")
