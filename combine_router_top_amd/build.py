"""Build libmoe.so in-tree for gfx950 with hipcc.

Usage: python -m combine_router_top_amd.build [--jobs N]

Each source is compiled to an object under ``combine_router_top_amd/_build``
(in parallel), then linked into ``combine_router_top_amd/libmoe.so``.  Always
recompiles (the build check must exercise the compiler).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "dispatch.hip", "expert_gemm.hip", "combine.hip", "tile_forward.hip", "moe_api.cpp"]
# measurement-only streaming-read probe, linked into a library of its own
PROBE_SOURCE = "hbm_read_probe.hip"
PROBE_LIB = os.path.join(PKG, "libhbm_probe.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
            "-Wno-unused-function", "-I" + os.path.join(os.path.dirname(PKG), "include")]


def device_flags():
    # keep packed-fp32 instructions out of the generated code
    return ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]


def compile_one(src: str, defs=(), build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + ["-D" + d for d in defs]
    if src.endswith(".hip"):
        cmd += device_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = True, defs=(), lib: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile and link.  ``defs`` are extra preprocessor definitions (tile-shape
    tuning knobs such as MOE_XG_NW=4); ``lib``/``build_dir`` redirect the output."""
    os.makedirs(build_dir, exist_ok=True)
    with_probe = lib == LIB
    srcs = SOURCES + ([PROBE_SOURCE] if with_probe else [])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: compile_one(s, defs, build_dir), srcs)))
    _link([objs[s] for s in SOURCES], lib, verbose)
    if with_probe:
        _link([objs[PROBE_SOURCE]], PROBE_LIB, verbose)
    return lib


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-D", dest="defs", action="append", default=[])
    ap.add_argument("--lib", default=LIB)
    ap.add_argument("--build-dir", default=BUILD)
    a = ap.parse_args()
    build(a.jobs, defs=a.defs, lib=a.lib, build_dir=a.build_dir)


if __name__ == "__main__":
    main()
