"""Python binding of the C ABI in include/harp.h, one function per entry point.

Argument marshalling only: every computation runs in the gfx950 kernels of
libharp.so.  torch supplies device memory and the current HIP stream; every
tensor argument must already live on the GPU (there is no CPU path).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import Schedule, check, lib

_DT = {torch.float32: _lib.HARP_F32, torch.bfloat16: _lib.HARP_BF16, torch.int8: _lib.HARP_I8,
       torch.float64: _lib.HARP_F64}
_BLK_NAME = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (the library has no CPU path)")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _rows_ld(t, d, name):
    if t.dim() != 2 or t.shape[1] != d:
        raise ValueError(f"{name} must be 2-D with {d} columns, got {tuple(t.shape)}")
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.shape[0], (t.stride(0) if t.shape[0] > 1 else d)


# ------------------------------------------------------------------ sizes
def harp_theta_count(schedule, d: int) -> int:
    return int(lib().harp_theta_count(ctypes.byref(Schedule.of(schedule)), d))


def harp_gauss_count(schedule, d: int) -> int:
    return int(lib().harp_gauss_count(ctypes.byref(Schedule.of(schedule)), d))


def harp_block_count(schedule, d: int) -> int:
    return int(lib().harp_block_count(ctypes.byref(Schedule.of(schedule)), d))


def harp_group_count(schedule, d: int) -> int:
    return int(lib().harp_group_count(ctypes.byref(Schedule.of(schedule)), d))


def harp_rotate_weight_workspace(d_out: int, d_in: int) -> int:
    return int(lib().harp_rotate_weight_workspace(d_out, d_in))


# ------------------------------------------------------------------ setup
def harp_materialize_blocks(schedule, d: int, theta: torch.Tensor, gauss: torch.Tensor | None,
                            block_dtype: str = "f32", blocks_out: torch.Tensor | None = None,
                            scales_out: torch.Tensor | None = None, stream=None):
    """Blocks B = Q(theta) G for every stage and group (fp64 on device), stored
    as 'f32', 'bf16' or 'i8' (+ fp32 scales).  Returns (blocks, scales|None)."""
    _dev(theta, "theta")
    _dev(gauss, "gauss")
    if theta.dtype != torch.float64 or (gauss is not None and gauss.dtype != torch.float64):
        raise TypeError("theta and gauss must be float64")
    if not theta.is_contiguous() or (gauss is not None and not gauss.is_contiguous()):
        raise ValueError("theta and gauss must be contiguous")
    tdt = _BLK_NAME[block_dtype]
    if blocks_out is None:
        blocks_out = torch.empty(harp_block_count(schedule, d), dtype=tdt, device=theta.device)
    if block_dtype == "i8" and scales_out is None:
        scales_out = torch.empty(harp_group_count(schedule, d), dtype=torch.float32, device=theta.device)
    _dev(blocks_out, "blocks_out")
    _dev(scales_out, "scales_out")
    check(lib().harp_materialize_blocks(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta),
                                        _ptr(gauss), _DT[tdt],
                                        _ptr(blocks_out), _ptr(scales_out), _stream(stream)))
    return blocks_out, (scales_out if block_dtype == "i8" else None)


def harp_quantize_theta(schedule, d: int, theta: torch.Tensor, codes_out: torch.Tensor | None = None,
                        scales_out: torch.Tensor | None = None, stream=None):
    """int8 codes and one fp32 scale per stage of fp64 theta, on device.
    Returns (codes, scales)."""
    _dev(theta, "theta")
    if theta.dtype != torch.float64 or not theta.is_contiguous():
        raise TypeError("theta must be contiguous float64")
    if codes_out is None:
        codes_out = torch.empty(harp_theta_count(schedule, d), dtype=torch.int8, device=theta.device)
    if scales_out is None:
        scales_out = torch.empty(len(tuple(schedule)), dtype=torch.float32, device=theta.device)
    _dev(codes_out, "codes_out")
    _dev(scales_out, "scales_out")
    check(lib().harp_quantize_theta(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta), _ptr(codes_out),
                                    _ptr(scales_out), _stream(stream)))
    return codes_out, scales_out


def harp_materialize_blocks_q8(schedule, d: int, theta_codes: torch.Tensor, theta_scales: torch.Tensor,
                               gauss: torch.Tensor | None, block_dtype: str = "f32",
                               blocks_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                               stream=None):
    """As harp_materialize_blocks, with theta given as int8 codes and one fp32
    scale per stage.  Returns (blocks, scales|None)."""
    _dev(theta_codes, "theta_codes")
    _dev(theta_scales, "theta_scales")
    _dev(gauss, "gauss")
    if theta_codes.dtype != torch.int8 or theta_scales.dtype != torch.float32:
        raise TypeError("theta_codes must be int8 and theta_scales float32")
    if gauss is not None and gauss.dtype != torch.float64:
        raise TypeError("gauss must be float64")
    if not theta_codes.is_contiguous() or not theta_scales.is_contiguous() or \
            (gauss is not None and not gauss.is_contiguous()):
        raise ValueError("theta_codes, theta_scales and gauss must be contiguous")
    if theta_codes.numel() != harp_theta_count(schedule, d) or \
            theta_scales.numel() != len(tuple(schedule)):
        raise ValueError("theta_codes / theta_scales have the wrong length for this schedule")
    tdt = _BLK_NAME[block_dtype]
    if blocks_out is None:
        blocks_out = torch.empty(harp_block_count(schedule, d), dtype=tdt, device=theta_codes.device)
    if block_dtype == "i8" and scales_out is None:
        scales_out = torch.empty(harp_group_count(schedule, d), dtype=torch.float32, device=theta_codes.device)
    _dev(blocks_out, "blocks_out")
    _dev(scales_out, "scales_out")
    check(lib().harp_materialize_blocks_q8(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta_codes),
                                           _ptr(theta_scales), _ptr(gauss), _DT[tdt], _ptr(blocks_out),
                                           _ptr(scales_out), _stream(stream)))
    return blocks_out, (scales_out if block_dtype == "i8" else None)


# ------------------------------------------------------------------ apply
def _apply(fn, schedule, d, blocks, scales, signs, x, y, stream):
    _dev(blocks, "blocks")
    _dev(scales, "scales")
    _dev(signs, "signs")
    _dev(x, "x")
    rows, ldx = _rows_ld(x, d, "x")
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y")
    rows_y, ldy = _rows_ld(y, d, "y")
    if rows_y != rows or y.dtype != x.dtype:
        raise ValueError("y must match x in rows and dtype")
    if signs is not None and signs.dtype != torch.int8:
        raise TypeError("signs must be int8")
    check(fn(ctypes.byref(Schedule.of(schedule)), d, _ptr(blocks), _DT[blocks.dtype], _ptr(scales),
             _ptr(signs), _ptr(x), ldx, _ptr(y), ldy, rows, _DT[x.dtype], _stream(stream)))
    return y


def harp_apply(schedule, d: int, blocks, scales, signs, x, y=None, stream=None):
    """y = S_{m-1} ... S_0 D_s x for every row of x (x, y: rows x d, f32/bf16)."""
    return _apply(lib().harp_apply, schedule, d, blocks, scales, signs, x, y, stream)


def harp_apply_inverse(schedule, d: int, blocks, scales, signs, y, x=None, stream=None):
    """x = D_s S_0^T ... S_{m-1}^T y for every row of y."""
    return _apply(lib().harp_apply_inverse, schedule, d, blocks, scales, signs, y, x, stream)


def harp_apply_decode_workspace(schedule, d: int, block_dtype: str, rows: int) -> int:
    """Workspace bytes harp_apply_decode needs (0: one launch, -1: unsupported)."""
    return int(lib().harp_apply_decode_workspace(ctypes.byref(Schedule.of(schedule)), d,
                                                 _DT[_BLK_NAME[block_dtype]], rows))


def harp_apply_decode(schedule, d: int, blocks, scales, signs, x, y=None, inverse: bool = False,
                      workspace=None, stream=None):
    """Small-batch apply (1 to a few hundred rows), forward or inverse.
    workspace: a device tensor of at least harp_apply_decode_workspace() bytes
    (allocated here when None and needed)."""
    _dev(blocks, "blocks")
    _dev(scales, "scales")
    _dev(signs, "signs")
    _dev(x, "x")
    _dev(workspace, "workspace")
    rows, ldx = _rows_ld(x, d, "x")
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y")
    rows_y, ldy = _rows_ld(y, d, "y")
    if rows_y != rows or y.dtype != x.dtype:
        raise ValueError("y must match x in rows and dtype")
    if signs is not None and signs.dtype != torch.int8:
        raise TypeError("signs must be int8")
    sch = Schedule.of(schedule)
    if workspace is None:
        need = int(lib().harp_apply_decode_workspace(ctypes.byref(sch), d, _DT[blocks.dtype], rows))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().harp_apply_decode(ctypes.byref(sch), d, _ptr(blocks), _DT[blocks.dtype], _ptr(scales),
                                  _ptr(signs), _ptr(x), ldx, _ptr(y), ldy, rows, _DT[x.dtype], int(inverse),
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def harp_apply_vjp_workspace(schedule, d: int, rows: int) -> int:
    """Workspace bytes harp_apply_vjp needs (-1: a radix above 8)."""
    return int(lib().harp_apply_vjp_workspace(ctypes.byref(Schedule.of(schedule)), d, rows))


def harp_apply_vjp(schedule, d: int, blocks, scales, signs, x, dy, dx=None, want_dx: bool = True,
                   dblocks=None, workspace=None, stream=None):
    """Reverse mode of harp_apply for an upstream gradient dy: returns
    (dx or None, dblocks), dblocks fp32 in the block layout."""
    for n, t in (("blocks", blocks), ("scales", scales), ("signs", signs), ("x", x), ("dy", dy),
                 ("dx", dx), ("dblocks", dblocks), ("workspace", workspace)):
        _dev(t, n)
    rows, ldx = _rows_ld(x, d, "x")
    rows_g, lddy = _rows_ld(dy, d, "dy")
    if rows_g != rows or dy.dtype != x.dtype:
        raise ValueError("dy must match x in rows and dtype")
    if signs is not None and signs.dtype != torch.int8:
        raise TypeError("signs must be int8")
    if dx is None and want_dx:
        dx = torch.empty_like(x)
    lddx = 0
    if dx is not None:
        rows_d, lddx = _rows_ld(dx, d, "dx")
        if rows_d != rows or dx.dtype != x.dtype:
            raise ValueError("dx must match x in rows and dtype")
    if dblocks is None:
        dblocks = torch.empty(harp_block_count(schedule, d), dtype=torch.float32, device=x.device)
    sch = Schedule.of(schedule)
    if workspace is None:
        need = int(lib().harp_apply_vjp_workspace(ctypes.byref(sch), d, rows))
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().harp_apply_vjp(ctypes.byref(sch), d, _ptr(blocks), _DT[blocks.dtype], _ptr(scales), _ptr(signs),
                               _ptr(x), ldx, _ptr(dy), lddy, _ptr(dx), lddx, rows, _DT[x.dtype], _ptr(dblocks),
                               _ptr(workspace), ws_bytes, _stream(stream)))
    return dx, dblocks


def harp_theta_vjp(schedule, d: int, theta: torch.Tensor, gauss, dblocks, dtheta=None, stream=None):
    """dL/dtheta (fp64, theta's layout) from dL/dB (fp32 block layout)."""
    for n, t in (("theta", theta), ("gauss", gauss), ("dblocks", dblocks), ("dtheta", dtheta)):
        _dev(t, n)
    if theta.dtype != torch.float64 or (gauss is not None and gauss.dtype != torch.float64):
        raise TypeError("theta and gauss must be float64")
    if dblocks.dtype != torch.float32 or dblocks.numel() != harp_block_count(schedule, d):
        raise ValueError("dblocks must be float32 with harp_block_count() elements")
    if dtheta is None:
        dtheta = torch.empty_like(theta)
    check(lib().harp_theta_vjp(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta), _ptr(gauss), _ptr(dblocks),
                               _ptr(dtheta), _stream(stream)))
    return dtheta


def harp_rotate_weight(su, blocks_u, scales_u, signs_u, sv, blocks_v, scales_v, signs_v, w,
                       w_out=None, inverse: bool = False, workspace=None, stream=None):
    """W_out = M_U W M_V^T (inverse: M_U^T W M_V); W is prod(su) x prod(sv)."""
    for n, t in (("blocks_u", blocks_u), ("blocks_v", blocks_v), ("scales_u", scales_u), ("scales_v", scales_v),
                 ("signs_u", signs_u), ("signs_v", signs_v), ("w", w), ("workspace", workspace)):
        _dev(t, n)
    if blocks_u.dtype != blocks_v.dtype:
        raise TypeError("blocks_u and blocks_v must share a dtype")
    d_out, d_in = w.shape
    _, ldw = _rows_ld(w, d_in, "w")
    if w_out is None:
        w_out = torch.empty_like(w)
    _dev(w_out, "w_out")
    _, ldo = _rows_ld(w_out, d_in, "w_out")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().harp_rotate_weight(
        ctypes.byref(Schedule.of(su)), _ptr(blocks_u), _ptr(scales_u), _ptr(signs_u),
        ctypes.byref(Schedule.of(sv)), _ptr(blocks_v), _ptr(scales_v), _ptr(signs_v),
        _DT[blocks_u.dtype], _ptr(w), ldw, _ptr(w_out), ldo, d_out, d_in, _DT[w.dtype], int(bool(inverse)),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return w_out


def rht_compose(schedule, d: int, signs, x, y=None, inverse: bool = False, stream=None):
    """y = (H D_k) ... (H D_1) x (inverse: (D_1 H) ... (D_k H) x); signs: k x d int8."""
    _dev(signs, "signs")
    _dev(x, "x")
    if signs.dtype != torch.int8 or signs.dim() != 2 or signs.shape[1] != d or not signs.is_contiguous():
        raise ValueError("signs must be a contiguous int8 tensor of shape (k, d)")
    rows, ldx = _rows_ld(x, d, "x")
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y")
    _, ldy = _rows_ld(y, d, "y")
    check(lib().rht_compose(ctypes.byref(Schedule.of(schedule)), d, _ptr(signs), signs.shape[0],
                            _ptr(x), ldx, _ptr(y), ldy, rows, _DT[x.dtype], int(bool(inverse)), _stream(stream)))
    return y
