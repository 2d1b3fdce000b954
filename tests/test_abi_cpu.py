"""Host-side tests of the C-ABI library (no GPU needed).

The library must load, export every function include/harp.h declares, size
its parameter arrays like the oracle, and reject malformed calls on the host
before any HIP call (so these calls are safe without a device).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import harp_oracle as O
from structured_rotations_amd import _lib
from structured_rotations_amd._lib import Schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "harp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(?:harp_status|int64_t|size_t|const char\*)\s+(\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_header_declares_the_abi():
    names = _declared_functions()
    for want in ("harp_apply", "harp_apply_inverse", "harp_rotate_weight", "rht_compose",
                 "harp_materialize_blocks", "harp_quantize_theta", "harp_materialize_blocks_q8",
                 "harp_status_str", "harp_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in harp.h but not exported"


@pytest.mark.parametrize("schedule", [(2,) * 6, (8, 8, 8, 8), (8, 8, 8, 5, 2), (8, 8, 8, 3, 3, 3), (8, 8, 8, 16),
                                      (3, 5, 7), (16, 2)])
def test_size_helpers_match_oracle(lib, schedule):
    d = int(np.prod(schedule))
    s = ctypes.byref(Schedule.of(schedule))
    assert lib.harp_theta_count(s, d) == sum(O.theta_counts(schedule, d))
    assert lib.harp_gauss_count(s, d) == sum(b * b for b in schedule if not O.is_pow2(b))
    assert lib.harp_block_count(s, d) == sum(d * b for b in schedule)
    assert lib.harp_group_count(s, d) == sum(d // b for b in schedule)


@pytest.mark.parametrize("schedule,d", [((8, 8), 65), ((1, 64), 64), ((17, 2), 34), ((2,) * 17, 2 ** 17),
                                        ((), 1), ((8, 8, 8, 8, 8, 8), 8 ** 6)])
def test_size_helpers_reject_bad_schedules(lib, schedule, d):
    sch = Schedule()
    sch.m = len(schedule)
    for i, b in enumerate(schedule[:16]):
        sch.radix[i] = b
    assert lib.harp_theta_count(ctypes.byref(sch), d) == -1


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000)


def _apply(lib, schedule=(8, 8), d=64, blocks=FAKE, bdt=_lib.HARP_F32, scales=None, signs=None, x=FAKE,
           ldx=64, y=FAKE2, ldy=64, rows=4, io=_lib.HARP_F32, inverse=False):
    fn = lib.harp_apply_inverse if inverse else lib.harp_apply
    return fn(ctypes.byref(Schedule.of(schedule)), d, blocks, bdt, scales, signs, x, ldx, y, ldy, rows, io, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=65), _lib.HARP_ERR_INVALID_ARG),                       # prod != d
    (dict(schedule=(8, 9), d=72, rows=-1), _lib.HARP_ERR_INVALID_ARG),
    (dict(ldx=32), _lib.HARP_ERR_INVALID_ARG),                     # ld < d
    (dict(x=None), _lib.HARP_ERR_INVALID_ARG),                     # NULL with rows > 0
    (dict(x=ctypes.c_void_p(0x10002)), _lib.HARP_ERR_INVALID_ARG),  # misaligned f32
    (dict(io=_lib.HARP_I8), _lib.HARP_ERR_UNSUPPORTED),
    (dict(io=_lib.HARP_F64), _lib.HARP_ERR_UNSUPPORTED),
    (dict(bdt=_lib.HARP_F64), _lib.HARP_ERR_UNSUPPORTED),
    (dict(bdt=_lib.HARP_I8), _lib.HARP_ERR_INVALID_ARG),           # int8 blocks without scales
    (dict(scales=FAKE), _lib.HARP_ERR_INVALID_ARG),                # scales with f32 blocks
    (dict(blocks=None), _lib.HARP_ERR_INVALID_ARG),
    (dict(y=ctypes.c_void_p(0x10000 + 64)), _lib.HARP_ERR_INVALID_ARG),  # partial overlap
    (dict(y=FAKE, ldy=128), _lib.HARP_ERR_INVALID_ARG),           # in place with different ld
    (dict(inverse=True, d=63), _lib.HARP_ERR_INVALID_ARG),
])
def test_apply_rejects_on_host(lib, kw, status):
    assert _apply(lib, **kw) == status
    assert lib.harp_last_error().decode() != ""


def test_apply_zero_rows_is_a_noop(lib):
    assert _apply(lib, rows=0, x=None, y=None) == _lib.HARP_OK


def test_oversized_schedule_struct_rejected(lib):
    sch = Schedule()
    sch.m = 17
    assert lib.harp_apply(ctypes.byref(sch), 64, FAKE, 0, None, None, FAKE, 64, FAKE2, 64, 1, 0, None) == \
        _lib.HARP_ERR_INVALID_ARG
    assert lib.harp_apply(None, 64, FAKE, 0, None, None, FAKE, 64, FAKE2, 64, 1, 0, None) == _lib.HARP_ERR_INVALID_ARG


def test_rht_rejects_on_host(lib):
    s = ctypes.byref(Schedule.of((8, 5)))
    assert lib.rht_compose(s, 40, FAKE, 3, FAKE, 40, FAKE2, 40, 2, 0, 0, None) == _lib.HARP_ERR_UNSUPPORTED
    s = ctypes.byref(Schedule.of((8, 8)))
    assert lib.rht_compose(s, 64, FAKE, 0, FAKE, 64, FAKE2, 64, 2, 0, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.rht_compose(s, 64, FAKE, 9, FAKE, 64, FAKE2, 64, 2, 0, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.rht_compose(s, 64, None, 3, FAKE, 64, FAKE2, 64, 2, 0, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.rht_compose(s, 64, None, 3, None, 64, None, 64, 0, 0, 0, None) == _lib.HARP_OK


def test_materialize_rejects_on_host(lib):
    s = ctypes.byref(Schedule.of((8, 5)))
    assert lib.harp_materialize_blocks(s, 40, FAKE, None, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.harp_materialize_blocks(s, 40, None, FAKE, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.harp_materialize_blocks(s, 40, FAKE, FAKE, 2, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert lib.harp_materialize_blocks(s, 40, FAKE, FAKE, 3, FAKE2, None, None) == _lib.HARP_ERR_UNSUPPORTED


def test_theta_i8_entry_points_reject_on_host(lib):
    s = ctypes.byref(Schedule.of((8, 5)))
    q8 = lib.harp_materialize_blocks_q8
    assert q8(s, 40, None, FAKE, FAKE, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert q8(s, 40, FAKE, None, FAKE, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert q8(s, 40, FAKE, FAKE, None, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert q8(s, 40, FAKE, FAKE, FAKE, 2, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert q8(s, 40, FAKE, FAKE, FAKE, 3, FAKE2, None, None) == _lib.HARP_ERR_UNSUPPORTED
    assert q8(s, 41, FAKE, FAKE, FAKE, 0, FAKE2, None, None) == _lib.HARP_ERR_INVALID_ARG
    qt = lib.harp_quantize_theta
    assert qt(s, 40, None, FAKE, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG
    assert qt(s, 40, FAKE, None, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG
    assert qt(s, 40, FAKE, FAKE, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert qt(s, 41, FAKE, FAKE, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG


def test_rotate_weight_rejects_on_host(lib):
    su = ctypes.byref(Schedule.of((8, 3)))
    sv = ctypes.byref(Schedule.of((8, 5)))
    args = dict(bu=FAKE, bv=FAKE, w=FAKE, ldw=40, wo=FAKE2, ldo=40, dout=24, din=40, ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return lib.harp_rotate_weight(su, a["bu"], None, None, sv, a["bv"], None, None, 0, a["w"], a["ldw"],
                                      a["wo"], a["ldo"], a["dout"], a["din"], 0, 0, a["ws"], a["wsb"], None)
    assert call(dout=25) == _lib.HARP_ERR_INVALID_ARG
    assert call(din=41) == _lib.HARP_ERR_INVALID_ARG
    assert call(ldw=39) == _lib.HARP_ERR_INVALID_ARG
    assert call(bu=None) == _lib.HARP_ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(0x40000), wsb=100) == _lib.HARP_ERR_INVALID_ARG      # too small
    assert call(ws=ctypes.c_void_p(0x40004), wsb=24 * 40 * 4) == _lib.HARP_ERR_INVALID_ARG  # misaligned
    assert lib.harp_rotate_weight_workspace(24, 40) == 24 * 40 * 4
    assert lib.harp_rotate_weight_workspace(0, 40) == 0


def test_status_strings(lib):
    assert lib.harp_status_str(0) == b"HARP_OK"
    assert lib.harp_status_str(-1) == b"HARP_ERR_INVALID_ARG"
    assert lib.harp_status_str(-2) == b"HARP_ERR_UNSUPPORTED"
    assert lib.harp_status_str(-3) == b"HARP_ERR_LAUNCH"
    assert lib.harp_version().startswith(b"harp-gfx950")


def test_decode_workspace_sizes_on_host(lib):
    ws = lib.harp_apply_decode_workspace
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 8))), 4096, _lib.HARP_F32, 3) == 3 * 4096 * 4
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 5, 2))), 5120, _lib.HARP_BF16, 64) == 64 * 5120 * 4
    assert ws(ctypes.byref(Schedule.of((8, 8))), 64, _lib.HARP_F32, 5) == 0      # one launch
    # above 128 rows the call runs the throughput row kernels: no hand-off buffer
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 8))), 4096, _lib.HARP_F32, 128) == 128 * 4096 * 4
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 8))), 4096, _lib.HARP_F32, 129) == 0
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 5, 2))), 5120, _lib.HARP_BF16, 1024) == 0
    assert ws(ctypes.byref(Schedule.of((8, 8))), 65, _lib.HARP_F32, 5) == -1     # not a factorisation
    assert ws(ctypes.byref(Schedule.of((8, 8))), 64, 7, 5) == -1                 # bad dtype
    # a size that does not fit in int64 is -1, not a wrapped number
    assert ws(ctypes.byref(Schedule.of((8, 8, 8, 8))), 4096, _lib.HARP_F32, 1 << 62) == -1


def test_row_extent_overflow_rejected_on_host(lib):
    # rows x leading dimension past the address space: an error, before any launch
    big = (1 << 62) // 4096
    assert _apply(lib, schedule=(8, 8), d=64, rows=big, ldx=1 << 40, ldy=1 << 40) == _lib.HARP_ERR_INVALID_ARG


def test_decode_rejects_on_host(lib):
    s = ctypes.byref(Schedule.of((8, 8, 8, 8)))
    dec = lib.harp_apply_decode
    # rows above the maximum
    assert dec(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 1025, 1, 0, FAKE, 1 << 30, None) == \
        _lib.HARP_ERR_INVALID_ARG
    # workspace missing / too small
    assert dec(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 2, 1, 0, None, 0, None) == \
        _lib.HARP_ERR_INVALID_ARG
    assert dec(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 2, 1, 0, FAKE, 2 * 4096 * 4 - 1, None) == \
        _lib.HARP_ERR_INVALID_ARG
    # int8 blocks without scales, bad io dtype
    assert dec(s, 4096, FAKE, 2, None, None, FAKE, 4096, FAKE2, 4096, 2, 1, 0, FAKE, 1 << 20, None) == \
        _lib.HARP_ERR_INVALID_ARG
    assert dec(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 2, 2, 0, FAKE, 1 << 20, None) == \
        _lib.HARP_ERR_UNSUPPORTED
    # above 128 rows no workspace is needed: a NULL one passes the host checks
    # (the call then fails only on an odd x, which no element size allows)
    assert dec(s, 4096, FAKE, 0, None, None, ctypes.c_void_p(0x10001), 4096, FAKE2, 4096, 200, 1, 0, None, 0,
               None) == _lib.HARP_ERR_INVALID_ARG
    assert "aligned" in lib.harp_last_error().decode()
    # zero rows: no launch, OK
    assert dec(s, 4096, None, 0, None, None, None, 4096, None, 4096, 0, 1, 0, None, 0, None) == _lib.HARP_OK


def test_vjp_rejects_on_host(lib):
    s = ctypes.byref(Schedule.of((8, 8, 8, 8)))
    need = lib.harp_apply_vjp_workspace(s, 4096, 5)
    assert need > 5 * 4096 * 4 * 5       # three activations + two gradient rows + partial sums
    assert lib.harp_apply_vjp_workspace(ctypes.byref(Schedule.of((16, 16))), 256, 5) == -1
    assert lib.harp_apply_vjp_workspace(s, 4096, 1 << 60) == -1      # size past int64
    vjp = lib.harp_apply_vjp
    args = lambda **kw: [s, 4096, kw.get("blocks", FAKE), kw.get("bdt", 0), kw.get("scales", None), None,
                         FAKE, 4096, FAKE2, 4096, kw.get("dx", None), 4096, kw.get("rows", 5), kw.get("io", 1),
                         kw.get("dblocks", FAKE), kw.get("ws", FAKE), kw.get("wsb", need), None]
    assert vjp(*args(ws=None)) == _lib.HARP_ERR_INVALID_ARG
    assert vjp(*args(wsb=need - 1)) == _lib.HARP_ERR_INVALID_ARG
    assert vjp(*args(dblocks=None)) == _lib.HARP_ERR_INVALID_ARG
    assert vjp(*args(rows=0)) == _lib.HARP_ERR_INVALID_ARG
    assert vjp(*args(bdt=2)) == _lib.HARP_ERR_INVALID_ARG          # int8 without scales
    assert vjp(*args(io=2)) == _lib.HARP_ERR_UNSUPPORTED
    s16 = ctypes.byref(Schedule.of((16, 16)))
    assert vjp(s16, 256, FAKE, 0, None, None, FAKE, 256, FAKE2, 256, None, 256, 5, 1, FAKE, FAKE, 1 << 20,
               None) == _lib.HARP_ERR_UNSUPPORTED
    tv = lib.harp_theta_vjp
    assert tv(s, 4096, None, None, FAKE, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG
    assert tv(s, 4096, FAKE, None, None, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG
    assert tv(s, 4096, FAKE, None, FAKE, None, None) == _lib.HARP_ERR_INVALID_ARG
    assert tv(ctypes.byref(Schedule.of((8, 5))), 40, FAKE, None, FAKE, FAKE2, None) == _lib.HARP_ERR_INVALID_ARG


def test_decode_noalloc_rejects_on_host(lib):
    na = lib.harp_apply_decode_noalloc
    s = ctypes.byref(Schedule.of((8, 8, 8, 8)))
    assert na(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 1025, 1, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert na(s, 4096, FAKE, 2, None, None, FAKE, 4096, FAKE2, 4096, 2, 1, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert na(s, 4096, FAKE, 0, None, None, FAKE, 4096, FAKE2, 4096, 2, 2, 0, None) == _lib.HARP_ERR_UNSUPPORTED
    # 128 rows of d = 32768 need 16 MiB of hand-off rows, beyond the 8 MiB buffer
    s5 = ctypes.byref(Schedule.of((8, 8, 8, 8, 8)))
    big = ctypes.c_void_p(1 << 40)
    assert na(s5, 32768, FAKE, 0, None, None, big, 32768, big, 32768, 128, 1, 0, None) == _lib.HARP_ERR_INVALID_ARG
    assert "HARP_NOALLOC_SCRATCH_BYTES" in lib.harp_last_error().decode()
    assert na(s, 4096, None, 0, None, None, None, 4096, None, 4096, 0, 1, 0, None) == _lib.HARP_OK
