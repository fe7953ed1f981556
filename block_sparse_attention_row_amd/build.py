"""Build libsparse_attn.so (HIP, gfx950) in-tree with hipcc.

    python -m block_sparse_attention_row_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
ARCH = os.environ.get("SPARSE_ATTN_ARCH", "gfx950")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-inline-asm",   # M0 is set inside the direct-load asm (the compiler never keeps values there)
    # device code sees no NaN inputs: max needs no canonicalising moves (host checks keep NaN semantics)
    "-Xarch_device", "-fno-honor-nans",
    # packed fp32 VALU forms stay off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build")
# the host pass does not know the packed-fp32 target feature; that warning is harmless
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + f".{os.getpid()}.o") for src in sources()]
    cmds = [["hipcc", *COMMON, "-c", src, "-o", obj] for src, obj in zip(sources(), objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))
    try:
        with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
            errs = list(ex.map(_run, cmds))
        tmp = LIB + f".tmp{os.getpid()}"
        errs.append(_run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
