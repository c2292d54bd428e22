"""Build libarepi.so (gfx950) from csrc/ with hipcc, in-tree.

Usage: python -m all_reduce_epilogues_amd.build [--isa DIR] [-j N]

--isa DIR keeps the compiler's intermediate files (including the gfx950
assembly) under DIR for inspection.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libarepi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "gemm_rs.hip", "gemm_rs_mixed.hip", "gemm_rs_ring.hip", "gemm_rs_fp8.hip", "lamport.hip", "combine.hip", "emu_producer.hip"]

# -packed-fp32-ops is turned off for every device compile: the compiler still
# vectorises, but never emits the packed fp32 add/mul/fma forms.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-strict-aliasing", "-Wall", "-Wno-unused-function",
]


def _compile(src: str, obj: str, isa_dir: str | None) -> str:
    cmd = [HIPCC, *FLAGS, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    cwd = None
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
        cmd.insert(1, "-save-temps")
        cwd = isa_dir
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return msg


def build(isa_dir: str | None = None, jobs: int = 8, verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, s, o, isa_dir) for s, o in zip(SOURCES, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None)
    ap.add_argument("-j", type=int, default=8)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.isa, a.j, a.v))


if __name__ == "__main__":
    main()
