"""Build libharp.so (gfx950) in-tree with hipcc.

    python -m structured_rotations_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only; the plain C++ planning layer is
compiled with the host compiler.  Packed fp32 VALU instructions are disabled
for the device code (-packed-fp32-ops).  Objects go to
structured_rotations_amd/_build/, the library to
structured_rotations_amd/libharp.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libharp.so")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
HIP_SOURCES = ["api.hip", "apply_tile.hip", "apply_mfma.hip", "apply_valu.hip", "apply_fast.hip", "rht.hip", "rotate_cols.hip", "col_dense.hip", "materialize.hip", "decode.hip", "vjp.hip"]
CXX_SOURCES = ["plan.cpp"]

DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC]


# The sources each measured kernel is built and launched from: a counter
# record stays valid while these files are unchanged.
KERNEL_SOURCES = {
    "apply_pipe": ["apply_fast.hip", "row_io.h", "common.h"],
    "apply_5120": ["apply_fast.hip", "row_io.h", "common.h"],
    "rht_wave": ["rht.hip", "common.h"],
    "col_pass": ["rotate_cols.hip", "col_dense.hip", "apply_fast.hip", "row_io.h", "common.h", "api.hip"],
}


def source_hash(kernel: str | None = None) -> str:
    """Hash of the sources of one measured kernel (KERNEL_SOURCES), or of every
    kernel and launcher source under csrc/ when no kernel is named."""
    import hashlib
    h = hashlib.sha256()
    files = KERNEL_SOURCES.get(kernel) if kernel else None
    if files is None:
        files = [f for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".h", ".cpp"))]
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


def _stale(src: str, obj: str) -> bool:
    """True if obj is missing or older than its source or any header it may
    include (every header under csrc/ and include/ counts)."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return any(os.path.getmtime(f) > t for f in deps)


def build(jobs: int = 8, verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source (incremental=True: only those whose object is
    stale) and link libharp.so."""
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        if not incremental or _stale(os.path.join(CSRC, src), obj):
            steps.append([HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    cxx = shutil.which("g++") or "c++"
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        if not incremental or _stale(os.path.join(CSRC, src), obj):
            steps.append([cxx, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(_run, steps))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


PROBE_SRC = os.path.join(PKG, "hwprobe.hip")
PROBE = os.path.join(PKG, "hwprobe")


def build_probe(verbose: bool = True) -> str:
    """Compile the device-rate probe (a standalone gfx950 program)."""
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", PROBE_SRC, "-o", PROBE])
    if verbose:
        print(f"built {PROBE}")
    return PROBE


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--incremental", action="store_true",
                    help="recompile only sources whose object is older than the source or a header")
    ap.add_argument("--probe", action="store_true", help="build the device-rate probe instead of the library")
    args = ap.parse_args()
    if args.probe:
        build_probe()
        return 0
    build(args.jobs, incremental=args.incremental)
    return 0


if __name__ == "__main__":
    sys.exit(main())
