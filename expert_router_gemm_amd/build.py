"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m expert_router_gemm_amd.build

Each source compiles to an object under expert_router_gemm_amd/_build/ in
parallel, then one shared library is linked next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["moe_api.cpp", "noalloc.hip", "eplb.cpp", "gemm_stream.hip", "gemm_tiled.hip",
           "route_topk.hip", "dispatch.hip", "combine.hip", "expert_counts.hip", "pack.hip"]

ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

# -Xclang -target-feature -Xclang -packed-fp32-ops: keep the compiler from
# forming packed fp32 VALU ops (the host pass prints a harmless warning).
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", CSRC, "-I", INCLUDE,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Per-file extra hipcc flags (none at present).
FILE_FLAGS = {}


def _compile(src: str, bdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPFLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = None, defines=(), build_dir: str = None) -> str:
    """Compile and link; ``out``/``defines``/``build_dir`` build a variant
    (e.g. another value of a compile-time tuning knob) elsewhere."""
    lib = out or LIB
    bdir = build_dir or BUILD
    os.makedirs(bdir, exist_ok=True)
    flags = [f"-D{d}" for d in defines]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, bdir, flags), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")


def build_probe(verbose: bool = False) -> str:
    """libmoe_probe.so: the HBM read-rate probe the benchmark reports beside
    the published peak (csrc/probe_read.hip; not part of libmoe)."""
    os.makedirs(BUILD, exist_ok=True)
    obj = _compile("probe_read.hip", BUILD, [])
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
    sys.exit(0)
