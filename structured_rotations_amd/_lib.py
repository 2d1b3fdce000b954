"""ctypes loader for libharp.so (the gfx950 C-ABI library in this package).

There is no fallback: if the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libharp.so")

HARP_OK = 0
HARP_ERR_INVALID_ARG = -1
HARP_ERR_UNSUPPORTED = -2
HARP_ERR_LAUNCH = -3

HARP_F32 = 0
HARP_BF16 = 1
HARP_I8 = 2
HARP_F64 = 3

MAX_STAGES = 16
NOALLOC_SCRATCH_BYTES = 8 << 20      # HARP_NOALLOC_SCRATCH_BYTES


class Schedule(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("radix", ctypes.c_int32 * MAX_STAGES)]

    @classmethod
    def of(cls, radices) -> "Schedule":
        """The (shared, read-only) struct for a radix list; the library copies
        it at call time, so one instance per schedule serves every call."""
        if isinstance(radices, Schedule):
            return radices
        key = tuple(int(b) for b in radices)
        s = _SCHEDULES.get(key)
        if s is None:
            if not 1 <= len(key) <= MAX_STAGES:
                raise ValueError(f"a schedule has 1..{MAX_STAGES} stages, got {len(key)}")
            s = cls()
            s.m = len(key)
            for i, b in enumerate(key):
                s.radix[i] = b
            _SCHEDULES[key] = s
        return s


_SCHEDULES: dict = {}


class HarpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIG = {
    "harp_theta_count": (_I64, [ctypes.POINTER(Schedule), _I64]),
    "harp_gauss_count": (_I64, [ctypes.POINTER(Schedule), _I64]),
    "harp_block_count": (_I64, [ctypes.POINTER(Schedule), _I64]),
    "harp_group_count": (_I64, [ctypes.POINTER(Schedule), _I64]),
    "harp_materialize_blocks": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _P, _I32, _P, _P, _P]),
    "harp_quantize_theta": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _P, _P, _P]),
    "harp_materialize_blocks_q8": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _P, _P, _I32, _P, _P, _P]),
    "harp_apply": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _P, _P, _I64, _P, _I64, _I64, _I32, _P]),
    "harp_apply_inverse": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _P, _P, _I64, _P, _I64, _I64,
                                  _I32, _P]),
    "harp_rotate_weight_workspace": (ctypes.c_size_t, [_I64, _I64]),
    "harp_apply_vjp_workspace": (_I64, [ctypes.POINTER(Schedule), _I64, _I64]),
    "harp_apply_vjp": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _P, _P, _I64, _P, _I64, _P, _I64, _I64,
                              _I32, _P, _P, ctypes.c_size_t, _P]),
    "harp_theta_vjp": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _P, _P, _P, _P]),
    "harp_apply_decode_workspace": (_I64, [ctypes.POINTER(Schedule), _I64, _I32, _I64]),
    "harp_apply_decode": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _P, _P, _I64, _P, _I64, _I64, _I32,
                                 _I32, _P, ctypes.c_size_t, _P]),
    "harp_apply_decode_noalloc": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _P, _P, _I64, _P, _I64,
                                         _I64, _I32, _I32, _P]),
    "harp_rotate_weight": (_I32, [ctypes.POINTER(Schedule), _P, _P, _P, ctypes.POINTER(Schedule), _P, _P, _P,
                                  _I32, _P, _I64, _P, _I64, _I64, _I64, _I32, _I32, _P, ctypes.c_size_t, _P]),
    "rht_compose": (_I32, [ctypes.POINTER(Schedule), _I64, _P, _I32, _P, _I64, _P, _I64, _I64, _I32, _I32, _P]),
    "harp_status_str": (ctypes.c_char_p, [_I32]),
    "harp_last_error": (ctypes.c_char_p, []),
    "harp_version": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m structured_rotations_amd.build` "
                        "(there is no CPU fallback)")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIG.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def check(status: int) -> None:
    if status != HARP_OK:
        msg = lib().harp_last_error().decode()
        name = lib().harp_status_str(status).decode()
        raise HarpError(status, f"{name}: {msg}")
