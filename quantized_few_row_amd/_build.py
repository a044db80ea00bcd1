"""Build ``librow_exact_mv.so`` in-tree with hipcc for gfx950.

Every HIP translation unit is compiled with packed-FP32 instruction
selection disabled and floating-point contraction off (all FMAs in the
kernels are explicit), then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librow_exact_mv.so")
ARCH = os.environ.get("ROW_EXACT_ARCH", "gfx950")

SOURCES = ["re_api.hip", "re_probe.hip", "re_norm.hip", "re_mv_f16.hip", "re_mv_q8_0.hip", "re_mv_q4_k.hip", "re_mv_q6_k.hip", "re_mv_q5_0.hip", "re_mv_f32.hip", "re_mv_bf16.hip"]
HEADERS = ["re_internal.h", "re_kernels.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=off", "-fno-fast-math", "-I", INCLUDE, "-I", CSRC]


def build(jobs: int = 6, verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile every HIP source (always) and link the shared library.

    ``out`` and ``defines`` (``NAME=VALUE`` macro overrides of the kernels'
    code-generation switches) build a variant library elsewhere, e.g. for an
    interleaved comparison with ``bench.py --ab``; the default is the
    product library next to this file."""
    objdir = BUILD if out == LIB else os.path.join(BUILD, os.path.basename(out) + ".objs")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cc = hipcc()
    flags = compile_flags() + [f"-D{d}" for d in defines]

    def one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-4000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr[-4000:]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build the row-exact mat-vec library for gfx950")
    ap.add_argument("-v", action="store_true", help="print the compile commands")
    ap.add_argument("--out", default=LIB, help="library path (default: the product library in the package)")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME=VALUE",
                    help="override a code-generation switch (a variant build; use with --out)")
    args = ap.parse_args()
    if args.defines and os.path.abspath(args.out) == LIB:
        raise SystemExit("_build: -D overrides build a variant; give it its own --out path")
    print(build(verbose=args.v, out=os.path.abspath(args.out), defines=tuple(args.defines)))
