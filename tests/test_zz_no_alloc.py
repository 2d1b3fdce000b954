"""harp_apply_decode_noalloc (the entry point for callers that cannot
allocate) against harp_apply_decode, through the C ABI.

Both run the same kernels; the no-alloc call keeps its hand-off rows in the
library's per-GPU buffer instead of a caller workspace, so its output must be
bit-identical to the workspace call's.  Two calls in a row, the second with a
smaller input (the buffer keeps the first call's rows, which the second must
not read), then a call above the row hand-over (no buffer needed) and one
that would need more than the buffer holds (rejected, nothing launched).
"""
import ctypes

import numpy as np
import pytest
import torch

from structured_rotations_amd import _lib, api
from structured_rotations_amd import inputs as I
from structured_rotations_amd._lib import Schedule

pytestmark = pytest.mark.gpu


def _case(sch, d, rows, io, blk, seed):
    g_sign, g_theta, _, g_data = I.streams(I.BASE_SEED + seed)
    theta = torch.from_numpy(I.theta_params(g_theta, sch, d, 0.05, 0.1)).cuda()
    gauss = I.gauss_mats(np.random.default_rng(seed), sch)
    gs = torch.from_numpy(gauss).cuda() if np.size(gauss) else None
    blocks, scales = api.harp_materialize_blocks(sch, d, theta, gs, blk)
    signs = torch.from_numpy(I.rademacher(g_sign, d)).cuda()
    x = torch.from_numpy(g_data.standard_t(3, size=(rows, d)).astype(np.float32))
    x = x.to(torch.bfloat16 if io == "bf16" else torch.float32).cuda()
    return blocks, scales, signs, x


def _noalloc(sch, d, blocks, scales, signs, x, y, inverse):
    ld = x.stride(0) if x.shape[0] > 1 else d
    return _lib.lib().harp_apply_decode_noalloc(
        ctypes.byref(Schedule.of(sch)), d, ctypes.c_void_p(blocks.data_ptr()), api._DT[blocks.dtype],
        None if scales is None else ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(signs.data_ptr()),
        ctypes.c_void_p(x.data_ptr()), ld, ctypes.c_void_p(y.data_ptr()), ld, x.shape[0], api._DT[x.dtype],
        int(inverse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("inverse", [False, True])
def test_noalloc_matches_workspace_call(inverse):
    # first call: 96 rows of d = 5120 (a two-launch schedule, 1.9 MiB of the
    # buffer); second call: 7 rows of d = 4096 (smaller), then 300 rows
    # (handed to the row kernels, no buffer)
    calls = [((8, 8, 8, 5, 2), 5120, 96, "bf16", "f32", 11), ((8, 8, 8, 8), 4096, 7, "f32", "bf16", 12),
             ((8, 8, 8, 8), 4096, 300, "bf16", "i8", 13)]
    for sch, d, rows, io, blk, seed in calls:
        print(f"\n[case] noalloc {sch} rows={rows} io={io} blocks={blk} inverse={inverse}", flush=True)
        blocks, scales, signs, x = _case(sch, d, rows, io, blk, seed)
        y_ref = api.harp_apply_decode(sch, d, blocks, scales, signs, x, inverse=inverse)
        y = torch.full_like(x, float("nan"))
        st = _noalloc(sch, d, blocks, scales, signs, x, y, inverse)
        assert st == _lib.HARP_OK, _lib.lib().harp_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"{sch} rows={rows}: no-alloc output differs from the workspace call"


def test_noalloc_binding_and_limit():
    sch, d = (8, 8, 8, 8), 4096
    blocks, scales, signs, x = _case(sch, d, 5, "bf16", "f32", 14)
    y = torch.empty_like(x)
    api.harp_apply_decode_noalloc(sch, d, blocks, scales, signs, x, y)
    ref = api.harp_apply_decode(sch, d, blocks, scales, signs, x)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    # 128 rows of d = 32768 would need 16 MiB of hand-off rows: rejected
    # before any launch (the buffer holds 8 MiB)
    sch2, d2 = (8, 8, 8, 8, 8), 32768
    assert _lib.lib().harp_apply_decode_workspace(ctypes.byref(Schedule.of(sch2)), d2, 0, 128) > \
        _lib.NOALLOC_SCRATCH_BYTES
    big = torch.empty((128, d2), dtype=torch.bfloat16, device="cuda")
    nb = api.harp_block_count(sch2, d2)
    st = _lib.lib().harp_apply_decode_noalloc(
        ctypes.byref(Schedule.of(sch2)), d2, ctypes.c_void_p(big.data_ptr()), _lib.HARP_F32, None, None,
        ctypes.c_void_p(big.data_ptr()), d2, ctypes.c_void_p(big.data_ptr()), d2, 128, _lib.HARP_BF16, 0, None)
    assert nb > 0 and st == _lib.HARP_ERR_INVALID_ARG
    assert "HARP_NOALLOC_SCRATCH_BYTES" in _lib.lib().harp_last_error().decode()
