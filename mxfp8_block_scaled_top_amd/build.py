"""Build libmoe_mi355x.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m mxfp8_block_scaled_top_amd.build [--jobs N] [--verbose]

Objects go to ``_build/`` at the repository root, the library to
``mxfp8_block_scaled_top_amd/_lib/libmoe_mi355x.so``.  Every call compiles
every source again.
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
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmoe_mi355x.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "router.hip", "permute.hip", "mxfp8.hip", "gemm.hip", "check.hip", "capi.cpp", "mlp.cpp", "linear.cpp", "trace.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 arithmetic stays off: only plain fp32 instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")


def _compile(src: str, verbose: bool, extra=(), odir: str = BUILD) -> str:
    obj = os.path.join(odir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if warn and verbose:
        print("\n".join(warn), file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = False, defines=(), out: str | None = None,
          objdir: str | None = None) -> str:
    """Compile every source and link the library (``out`` defaults to the
    in-tree path; ``defines`` are extra -D flags)."""
    lib_path = out or LIB
    odir = objdir or BUILD
    os.makedirs(odir, exist_ok=True)
    os.makedirs(os.path.dirname(lib_path), exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, odir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=None)
    ap.add_argument("--objdir", default=None)
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.defines, a.out, a.objdir))


if __name__ == "__main__":
    main()
