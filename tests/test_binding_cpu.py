"""Host-side checks of the Python binding (no GPU needed).

The C ABI receives bare pointers, one row count and one I/O dtype, so the
binding must reject, before it calls the library, every tensor whose size,
dtype or layout the kernels would misread: a short output, an output of
another dtype, parameter arrays of the wrong length or dtype, non-contiguous
parameter views.  These tests pass CPU tensors and replace the library's
transform entry points with a guard that fails if reached, so each case shows
that the check fires first (a well-formed call gets as far as the GPU-tensor
check, the last one before the library call).
"""
import numpy as np
import pytest
import torch

from oracle import harp_oracle as O
from structured_rotations_amd import api

SCH, D = (8, 5, 2), 80


class _Guard:
    """Forwards the size helpers to the real library; any other entry point
    fails the test."""

    SIZES = {"harp_theta_count", "harp_gauss_count", "harp_block_count", "harp_group_count",
             "harp_rotate_weight_workspace", "harp_apply_decode_workspace", "harp_apply_vjp_workspace",
             "harp_status_str", "harp_last_error"}

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in self.SIZES:
            return getattr(self._real, name)

        def launched(*a, **k):
            raise AssertionError(f"{name} reached the library")
        return launched


@pytest.fixture(autouse=True)
def guard(monkeypatch):
    real = api.lib()
    monkeypatch.setattr(api, "lib", lambda: _Guard(real))


def _params(schedule=SCH, d=D, blk=torch.float32):
    nb = sum(d * b for b in schedule)
    blocks = torch.zeros(nb, dtype=blk)
    scales = torch.ones(sum(d // b for b in schedule), dtype=torch.float32) if blk == torch.int8 else None
    signs = torch.ones(d, dtype=torch.int8)
    return blocks, scales, signs


def _gpu_only(fn):
    with pytest.raises(TypeError, match="GPU tensor"):
        fn()


def test_counts_match_the_oracle():
    assert api.harp_block_count(SCH, D) == sum(D * b for b in SCH)
    assert api.harp_group_count(SCH, D) == sum(D // b for b in SCH)
    assert api.harp_theta_count(SCH, D) == sum(O.theta_counts(SCH, D))


@pytest.mark.parametrize("fn", [api.harp_apply, api.harp_apply_inverse, api.harp_apply_decode])
def test_apply_calls_check_every_argument(fn):
    blocks, scales, signs = _params()
    x = torch.zeros(5, D, dtype=torch.bfloat16)
    _gpu_only(lambda: fn(SCH, D, blocks, scales, signs, x))                         # well formed
    with pytest.raises(ValueError, match="rows and dtype"):
        fn(SCH, D, blocks, scales, signs, x, torch.zeros(4, D, dtype=torch.bfloat16))   # short output
    with pytest.raises(ValueError, match="rows and dtype"):
        fn(SCH, D, blocks, scales, signs, x, torch.zeros(5, D, dtype=torch.float32))    # f32 out for bf16 in
    with pytest.raises(ValueError, match="elements"):
        fn(SCH, D, blocks[:-1], scales, signs, x)                                   # short blocks
    with pytest.raises(ValueError, match="contiguous"):
        fn(SCH, D, torch.zeros(2 * blocks.numel())[::2], scales, signs, x)          # strided view
    with pytest.raises(TypeError):
        fn(SCH, D, blocks.double(), scales, signs, x)                               # f64 blocks
    with pytest.raises(ValueError, match="elements"):
        fn(SCH, D, blocks, scales, signs[:-1], x)                                   # short signs
    with pytest.raises(TypeError):
        fn(SCH, D, blocks, scales, signs.float(), x)                                # signs not int8
    b8, s8, _ = _params(blk=torch.int8)
    with pytest.raises(ValueError, match="need scales"):
        fn(SCH, D, b8, None, signs, x)                                              # int8 without scales
    with pytest.raises(ValueError, match="elements"):
        fn(SCH, D, b8, s8[:-1], signs, x)                                           # short scales
    with pytest.raises(ValueError, match="int8 blocks only"):
        fn(SCH, D, blocks, s8, signs, x)                                            # scales with f32 blocks
    with pytest.raises(ValueError, match="columns"):
        fn(SCH, D, blocks, scales, signs, torch.zeros(5, D + 1, dtype=torch.bfloat16))


def test_rht_compose_checks_its_output():
    s = torch.ones(3, 64, dtype=torch.int8)
    x = torch.zeros(7, 64, dtype=torch.bfloat16)
    _gpu_only(lambda: api.rht_compose((8, 8), 64, s, x))
    with pytest.raises(ValueError, match="rows and dtype"):
        api.rht_compose((8, 8), 64, s, x, torch.zeros(6, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="rows and dtype"):
        api.rht_compose((8, 8), 64, s, x, torch.zeros(7, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        api.rht_compose((8, 8), 64, s[:, :63], x)


def test_rotate_weight_checks_its_output_and_parameters():
    su, du = (4, 3), 12
    bu, _, sgu = _params(su, du)
    bv, _, sgv = _params()
    w = torch.zeros(du, D, dtype=torch.bfloat16)
    _gpu_only(lambda: api.harp_rotate_weight(su, bu, None, sgu, SCH, bv, None, sgv, w))
    with pytest.raises(ValueError, match="shape and dtype"):
        api.harp_rotate_weight(su, bu, None, sgu, SCH, bv, None, sgv, w, torch.zeros(du - 1, D, dtype=w.dtype))
    with pytest.raises(ValueError, match="shape and dtype"):
        api.harp_rotate_weight(su, bu, None, sgu, SCH, bv, None, sgv, w, torch.zeros(du, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="blocks_u"):
        api.harp_rotate_weight(su, bu[:-1], None, sgu, SCH, bv, None, sgv, w)
    with pytest.raises(ValueError, match="signs_v"):
        api.harp_rotate_weight(su, bu, None, sgu, SCH, bv, None, sgv[:-1], w)
    with pytest.raises(TypeError, match="share a dtype"):
        api.harp_rotate_weight(su, bu, None, sgu, SCH, bv.bfloat16(), None, sgv, w)


def test_materialize_checks_every_array():
    nt = api.harp_theta_count(SCH, D)
    theta = torch.zeros(nt, dtype=torch.float64)
    gauss = torch.zeros(25, dtype=torch.float64)
    _gpu_only(lambda: api.harp_materialize_blocks(SCH, D, theta, gauss, "f32"))
    with pytest.raises(ValueError, match="elements"):
        api.harp_materialize_blocks(SCH, D, theta[:-1], gauss, "f32")
    with pytest.raises(ValueError, match="elements"):
        api.harp_materialize_blocks(SCH, D, theta, gauss[:-1], "f32")
    with pytest.raises(TypeError):
        api.harp_materialize_blocks(SCH, D, theta.float(), gauss, "f32")
    # a bf16 output for f32 blocks would be written past its end
    out = torch.zeros(api.harp_block_count(SCH, D), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        api.harp_materialize_blocks(SCH, D, theta, gauss, "f32", blocks_out=out)
    with pytest.raises(ValueError, match="elements"):
        api.harp_materialize_blocks(SCH, D, theta, gauss, "f32", blocks_out=torch.zeros(out.numel() - 1))
    with pytest.raises(ValueError, match="elements"):
        api.harp_materialize_blocks(SCH, D, theta, gauss, "i8", scales_out=torch.zeros(3))
    codes = torch.zeros(nt, dtype=torch.int8)
    with pytest.raises(ValueError, match="elements"):
        api.harp_materialize_blocks_q8(SCH, D, codes[:-1], torch.zeros(len(SCH)), gauss)
    with pytest.raises(ValueError, match="elements"):
        api.harp_quantize_theta(SCH, D, theta, codes_out=codes[:-1])


def test_vjp_checks_gradients():
    blocks, scales, signs = _params()
    x = torch.zeros(5, D, dtype=torch.float32)
    dy = torch.zeros(5, D, dtype=torch.float32)
    _gpu_only(lambda: api.harp_apply_vjp(SCH, D, blocks, scales, signs, x, dy))
    with pytest.raises(ValueError, match="rows and dtype"):
        api.harp_apply_vjp(SCH, D, blocks, scales, signs, x, dy[:4])
    with pytest.raises(ValueError, match="rows and dtype"):
        api.harp_apply_vjp(SCH, D, blocks, scales, signs, x, dy, dx=torch.zeros(5, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="elements"):
        api.harp_apply_vjp(SCH, D, blocks, scales, signs, x, dy, dblocks=torch.zeros(blocks.numel() - 1))
    nt = api.harp_theta_count(SCH, D)
    theta = torch.zeros(nt, dtype=torch.float64)
    with pytest.raises(ValueError, match="elements"):
        api.harp_theta_vjp(SCH, D, theta, torch.zeros(25, dtype=torch.float64), torch.zeros(blocks.numel() + 1))
    with pytest.raises(ValueError, match="elements"):
        api.harp_theta_vjp(SCH, D, theta, torch.zeros(25, dtype=torch.float64), torch.zeros(blocks.numel()),
                           dtheta=torch.zeros(nt - 1, dtype=torch.float64))


def test_bad_schedule_is_rejected_before_the_library():
    blocks, scales, signs = _params()
    with pytest.raises(ValueError, match="does not factor"):
        api.harp_apply((8, 5, 3), D, blocks, scales, signs, torch.zeros(2, D))
