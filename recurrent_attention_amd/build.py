"""Build liblinattn.so (gfx950) in-tree from ``csrc/``.

Every ``csrc/*.hip`` file is compiled by hipcc into ``_build/`` (in parallel)
and the objects are linked into ``recurrent_attention_amd/liblinattn.so``.
``python -m recurrent_attention_amd.build`` rebuilds everything;
``--incremental`` skips objects newer than their sources and headers.
``--check-hazards`` also compiles each source to device assembly and checks
every path from a matrix-core instruction to the first reader of its result
(:mod:`recurrent_attention_amd.hazards`); a violation fails the build.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h")))


def _compile(src, incremental, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(f) for f in [src] + _headers())
        if os.path.getmtime(obj) >= newest:
            return obj
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    return obj


def build(incremental: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    """Compile all kernels for gfx950 and link ``liblinattn.so``; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _assemble(src, out_dir):
    asm = os.path.join(out_dir, os.path.basename(src)[:-4] + ".s")
    cmd = [HIPCC] + CFLAGS + ["--cuda-device-only", "-S", src, "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {os.path.basename(src)}:\n{res.stderr}")
    return asm


def device_assembly(out_dir: str | None = None, jobs: int | None = None) -> list:
    """Compile every source to gfx950 assembly (same flags as the library)."""
    out_dir = out_dir or os.path.join(BUILD, "asm")
    os.makedirs(out_dir, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        return list(ex.map(lambda s: _assemble(s, out_dir), srcs))


def check_hazards(out_dir: str | None = None, jobs: int | None = None) -> list:
    """Violations (see :mod:`.hazards`) over the assembly of every source."""
    from . import hazards
    found = []
    for path in device_assembly(out_dir, jobs):
        with open(path) as f:
            found += [(os.path.basename(path), v) for v in hazards.check_asm(f.read())]
    return found


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--check-hazards", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.incremental, a.jobs, a.verbose))
    if a.check_hazards:
        found = check_hazards(jobs=a.jobs)
        for name, v in found:
            print(f"{name}: {v}")
        print(f"{len(found)} matrix-core hazard(s)")
        return 1 if found else 0
    return 0


if __name__ == "__main__":
    sys.exit(main())
