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


def _flat(t, name, dtype, count):
    """A parameter array: the given dtype, contiguous, exactly count elements
    (the C side receives only a pointer and cannot check any of this)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if count < 0:
        raise ValueError(f"{name}: the schedule does not factor d")
    if t.numel() != count:
        raise ValueError(f"{name} has {t.numel()} elements, the schedule needs {count}")


def _block_params(schedule, d, blocks, scales, signs, name=""):
    """blocks (f32/bf16/i8, harp_block_count elements), scales (fp32, one per
    group, with int8 blocks only) and signs (d int8, or None)."""
    if not isinstance(blocks, torch.Tensor) or blocks.dtype not in (torch.float32, torch.bfloat16, torch.int8):
        raise TypeError(f"blocks{name} must be a float32, bfloat16 or int8 tensor")
    _flat(blocks, "blocks" + name, blocks.dtype, harp_block_count(schedule, d))
    if blocks.dtype == torch.int8:
        if scales is None:
            raise ValueError(f"int8 blocks{name} need scales{name}")
        _flat(scales, "scales" + name, torch.float32, harp_group_count(schedule, d))
    elif scales is not None:
        raise ValueError(f"scales{name} go with int8 blocks only")
    if signs is not None:
        _flat(signs, "signs" + name, torch.int8, d)


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
    _flat(theta, "theta", torch.float64, harp_theta_count(schedule, d))
    if gauss is not None:
        _flat(gauss, "gauss", torch.float64, harp_gauss_count(schedule, d))
    tdt = _BLK_NAME[block_dtype]
    if blocks_out is None:
        blocks_out = torch.empty(harp_block_count(schedule, d), dtype=tdt, device=theta.device)
    if block_dtype == "i8" and scales_out is None:
        scales_out = torch.empty(harp_group_count(schedule, d), dtype=torch.float32, device=theta.device)
    _flat(blocks_out, "blocks_out", tdt, harp_block_count(schedule, d))
    if block_dtype == "i8":
        _flat(scales_out, "scales_out", torch.float32, harp_group_count(schedule, d))
    elif scales_out is not None:
        raise ValueError("scales_out goes with int8 blocks only")
    for n, t in (("theta", theta), ("gauss", gauss), ("blocks_out", blocks_out), ("scales_out", scales_out)):
        _dev(t, n)
    check(lib().harp_materialize_blocks(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta),
                                        _ptr(gauss), _DT[tdt],
                                        _ptr(blocks_out), _ptr(scales_out), _stream(stream)))
    return blocks_out, (scales_out if block_dtype == "i8" else None)


def harp_quantize_theta(schedule, d: int, theta: torch.Tensor, codes_out: torch.Tensor | None = None,
                        scales_out: torch.Tensor | None = None, stream=None):
    """int8 codes and one fp32 scale per stage of fp64 theta, on device.
    Returns (codes, scales)."""
    _flat(theta, "theta", torch.float64, harp_theta_count(schedule, d))
    if codes_out is None:
        codes_out = torch.empty(harp_theta_count(schedule, d), dtype=torch.int8, device=theta.device)
    if scales_out is None:
        scales_out = torch.empty(len(tuple(schedule)), dtype=torch.float32, device=theta.device)
    _flat(codes_out, "codes_out", torch.int8, harp_theta_count(schedule, d))
    _flat(scales_out, "scales_out", torch.float32, len(tuple(schedule)))
    for n, t in (("theta", theta), ("codes_out", codes_out), ("scales_out", scales_out)):
        _dev(t, n)
    check(lib().harp_quantize_theta(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta), _ptr(codes_out),
                                    _ptr(scales_out), _stream(stream)))
    return codes_out, scales_out


def harp_materialize_blocks_q8(schedule, d: int, theta_codes: torch.Tensor, theta_scales: torch.Tensor,
                               gauss: torch.Tensor | None, block_dtype: str = "f32",
                               blocks_out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None,
                               stream=None):
    """As harp_materialize_blocks, with theta given as int8 codes and one fp32
    scale per stage.  Returns (blocks, scales|None)."""
    _flat(theta_codes, "theta_codes", torch.int8, harp_theta_count(schedule, d))
    _flat(theta_scales, "theta_scales", torch.float32, len(tuple(schedule)))
    if gauss is not None:
        _flat(gauss, "gauss", torch.float64, harp_gauss_count(schedule, d))
    tdt = _BLK_NAME[block_dtype]
    if blocks_out is None:
        blocks_out = torch.empty(harp_block_count(schedule, d), dtype=tdt, device=theta_codes.device)
    if block_dtype == "i8" and scales_out is None:
        scales_out = torch.empty(harp_group_count(schedule, d), dtype=torch.float32, device=theta_codes.device)
    _flat(blocks_out, "blocks_out", tdt, harp_block_count(schedule, d))
    if block_dtype == "i8":
        _flat(scales_out, "scales_out", torch.float32, harp_group_count(schedule, d))
    elif scales_out is not None:
        raise ValueError("scales_out goes with int8 blocks only")
    for n, t in (("theta_codes", theta_codes), ("theta_scales", theta_scales), ("gauss", gauss),
                 ("blocks_out", blocks_out), ("scales_out", scales_out)):
        _dev(t, n)
    check(lib().harp_materialize_blocks_q8(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta_codes),
                                           _ptr(theta_scales), _ptr(gauss), _DT[tdt], _ptr(blocks_out),
                                           _ptr(scales_out), _stream(stream)))
    return blocks_out, (scales_out if block_dtype == "i8" else None)


# ------------------------------------------------------------------ apply
# Every call below checks shapes, dtypes and sizes first and that every tensor
# is on the GPU last, then calls the library once: nothing is launched for a
# call that fails a check.

def _out_like(out, x, d, name):
    """The output of a row transform: x's row count and dtype (the library is
    given one row count and one I/O dtype for both)."""
    if out is None:
        return torch.empty_like(x)
    rows, _ = _rows_ld(out, d, name)
    if rows != x.shape[0] or out.dtype != x.dtype:
        raise ValueError(f"{name} must match the input in rows and dtype: {tuple(out.shape)} {out.dtype} "
                         f"for {tuple(x.shape)} {x.dtype}")
    return out


def _apply(fn, schedule, d, blocks, scales, signs, x, y, stream):
    _block_params(schedule, d, blocks, scales, signs)
    rows, ldx = _rows_ld(x, d, "x")
    y = _out_like(y, x, d, "y")
    _, ldy = _rows_ld(y, d, "y")
    for n, t in (("blocks", blocks), ("scales", scales), ("signs", signs), ("x", x), ("y", y)):
        _dev(t, n)
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
    """Workspace bytes harp_apply_decode needs (0: none, -1: unsupported)."""
    return int(lib().harp_apply_decode_workspace(ctypes.byref(Schedule.of(schedule)), d,
                                                 _DT[_BLK_NAME[block_dtype]], rows))


def _workspace_bytes(workspace):
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    return workspace.numel() * workspace.element_size()


def harp_apply_decode(schedule, d: int, blocks, scales, signs, x, y=None, inverse: bool = False,
                      workspace=None, stream=None):
    """Small-batch apply (1 to a few hundred rows), forward or inverse.
    workspace: a device tensor of at least harp_apply_decode_workspace() bytes
    (allocated here when None and needed)."""
    _block_params(schedule, d, blocks, scales, signs)
    rows, ldx = _rows_ld(x, d, "x")
    y = _out_like(y, x, d, "y")
    _, ldy = _rows_ld(y, d, "y")
    sch = Schedule.of(schedule)
    if workspace is None:
        need = int(lib().harp_apply_decode_workspace(ctypes.byref(sch), d, _DT[blocks.dtype], rows))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = _workspace_bytes(workspace)
    for n, t in (("blocks", blocks), ("scales", scales), ("signs", signs), ("x", x), ("y", y),
                 ("workspace", workspace)):
        _dev(t, n)
    check(lib().harp_apply_decode(ctypes.byref(sch), d, _ptr(blocks), _DT[blocks.dtype], _ptr(scales),
                                  _ptr(signs), _ptr(x), ldx, _ptr(y), ldy, rows, _DT[x.dtype], int(inverse),
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def harp_apply_decode_noalloc(schedule, d: int, blocks, scales, signs, x, y, inverse: bool = False, stream=None):
    """harp_apply_decode with its hand-off rows in the library's own per-GPU
    buffer: allocates nothing (y must be given).  Calls that overlap in time
    on one GPU must not be issued (they share the buffer)."""
    _block_params(schedule, d, blocks, scales, signs)
    rows, ldx = _rows_ld(x, d, "x")
    if y is None:
        raise ValueError("y is required (this entry point allocates nothing)")
    y = _out_like(y, x, d, "y")
    _, ldy = _rows_ld(y, d, "y")
    for n, t in (("blocks", blocks), ("scales", scales), ("signs", signs), ("x", x), ("y", y)):
        _dev(t, n)
    check(lib().harp_apply_decode_noalloc(ctypes.byref(Schedule.of(schedule)), d, _ptr(blocks), _DT[blocks.dtype],
                                          _ptr(scales), _ptr(signs), _ptr(x), ldx, _ptr(y), ldy, rows,
                                          _DT[x.dtype], int(inverse), _stream(stream)))
    return y


def harp_apply_vjp_workspace(schedule, d: int, rows: int) -> int:
    """Workspace bytes harp_apply_vjp needs (-1: a radix above 8)."""
    return int(lib().harp_apply_vjp_workspace(ctypes.byref(Schedule.of(schedule)), d, rows))


def harp_apply_vjp(schedule, d: int, blocks, scales, signs, x, dy, dx=None, want_dx: bool = True,
                   dblocks=None, workspace=None, stream=None):
    """Reverse mode of harp_apply for an upstream gradient dy: returns
    (dx or None, dblocks), dblocks fp32 in the block layout."""
    _block_params(schedule, d, blocks, scales, signs)
    rows, ldx = _rows_ld(x, d, "x")
    if dy is None:
        raise ValueError("dy is required")
    dy = _out_like(dy, x, d, "dy")
    _, lddy = _rows_ld(dy, d, "dy")
    if dx is None and want_dx:
        dx = torch.empty_like(x)
    lddx = 0
    if dx is not None:
        dx = _out_like(dx, x, d, "dx")
        _, lddx = _rows_ld(dx, d, "dx")
    if dblocks is None:
        dblocks = torch.empty(harp_block_count(schedule, d), dtype=torch.float32, device=x.device)
    _flat(dblocks, "dblocks", torch.float32, harp_block_count(schedule, d))
    sch = Schedule.of(schedule)
    if workspace is None:
        need = int(lib().harp_apply_vjp_workspace(ctypes.byref(sch), d, rows))
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    ws_bytes = _workspace_bytes(workspace)
    for n, t in (("blocks", blocks), ("scales", scales), ("signs", signs), ("x", x), ("dy", dy),
                 ("dx", dx), ("dblocks", dblocks), ("workspace", workspace)):
        _dev(t, n)
    check(lib().harp_apply_vjp(ctypes.byref(sch), d, _ptr(blocks), _DT[blocks.dtype], _ptr(scales), _ptr(signs),
                               _ptr(x), ldx, _ptr(dy), lddy, _ptr(dx), lddx, rows, _DT[x.dtype], _ptr(dblocks),
                               _ptr(workspace), ws_bytes, _stream(stream)))
    return dx, dblocks


def harp_theta_vjp(schedule, d: int, theta: torch.Tensor, gauss, dblocks, dtheta=None, stream=None):
    """dL/dtheta (fp64, theta's layout) from dL/dB (fp32 block layout)."""
    _flat(theta, "theta", torch.float64, harp_theta_count(schedule, d))
    if gauss is not None:
        _flat(gauss, "gauss", torch.float64, harp_gauss_count(schedule, d))
    _flat(dblocks, "dblocks", torch.float32, harp_block_count(schedule, d))
    if dtheta is None:
        dtheta = torch.empty_like(theta)
    _flat(dtheta, "dtheta", torch.float64, harp_theta_count(schedule, d))
    for n, t in (("theta", theta), ("gauss", gauss), ("dblocks", dblocks), ("dtheta", dtheta)):
        _dev(t, n)
    check(lib().harp_theta_vjp(ctypes.byref(Schedule.of(schedule)), d, _ptr(theta), _ptr(gauss), _ptr(dblocks),
                               _ptr(dtheta), _stream(stream)))
    return dtheta


def harp_rotate_weight(su, blocks_u, scales_u, signs_u, sv, blocks_v, scales_v, signs_v, w,
                       w_out=None, inverse: bool = False, workspace=None, fp32_intermediates: bool = True,
                       stream=None):
    """W_out = M_U W M_V^T (inverse: M_U^T W M_V); W is prod(su) x prod(sv).

    Between its passes the rotation keeps the intermediate weight in fp32 in a
    workspace (allocated here when none is given).  fp32_intermediates=False
    with no workspace keeps it in W's dtype instead (no extra memory; for bf16
    W, three roundings in place of one)."""
    if w.dim() != 2:
        raise ValueError(f"w must be 2-D, got {tuple(w.shape)}")
    d_out, d_in = w.shape
    _block_params(su, d_out, blocks_u, scales_u, signs_u, "_u")
    _block_params(sv, d_in, blocks_v, scales_v, signs_v, "_v")
    if blocks_u.dtype != blocks_v.dtype:
        raise TypeError("blocks_u and blocks_v must share a dtype")
    _, ldw = _rows_ld(w, d_in, "w")
    if w_out is None:
        w_out = torch.empty_like(w)
    if tuple(w_out.shape) != tuple(w.shape) or w_out.dtype != w.dtype:
        raise ValueError(f"w_out must match w in shape and dtype: {tuple(w_out.shape)} {w_out.dtype} "
                         f"for {tuple(w.shape)} {w.dtype}")
    _, ldo = _rows_ld(w_out, d_in, "w_out")
    if workspace is None and fp32_intermediates:
        need = harp_rotate_weight_workspace(d_out, d_in)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    ws_bytes = _workspace_bytes(workspace)
    for n, t in (("blocks_u", blocks_u), ("blocks_v", blocks_v), ("scales_u", scales_u), ("scales_v", scales_v),
                 ("signs_u", signs_u), ("signs_v", signs_v), ("w", w), ("w_out", w_out),
                 ("workspace", workspace)):
        _dev(t, n)
    check(lib().harp_rotate_weight(
        ctypes.byref(Schedule.of(su)), _ptr(blocks_u), _ptr(scales_u), _ptr(signs_u),
        ctypes.byref(Schedule.of(sv)), _ptr(blocks_v), _ptr(scales_v), _ptr(signs_v),
        _DT[blocks_u.dtype], _ptr(w), ldw, _ptr(w_out), ldo, d_out, d_in, _DT[w.dtype], int(bool(inverse)),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return w_out


def rht_compose(schedule, d: int, signs, x, y=None, inverse: bool = False, stream=None):
    """y = (H D_k) ... (H D_1) x (inverse: (D_1 H) ... (D_k H) x); signs: k x d int8."""
    if not isinstance(signs, torch.Tensor) or signs.dtype != torch.int8 or signs.dim() != 2 or \
            signs.shape[1] != d or not signs.is_contiguous():
        raise ValueError("signs must be a contiguous int8 tensor of shape (k, d)")
    rows, ldx = _rows_ld(x, d, "x")
    y = _out_like(y, x, d, "y")
    _, ldy = _rows_ld(y, d, "y")
    for n, t in (("signs", signs), ("x", x), ("y", y)):
        _dev(t, n)
    check(lib().rht_compose(ctypes.byref(Schedule.of(schedule)), d, _ptr(signs), signs.shape[0],
                            _ptr(x), ldx, _ptr(y), ldy, rows, _DT[x.dtype], int(bool(inverse)), _stream(stream)))
    return y
