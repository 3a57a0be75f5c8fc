"""Build libqsmoe.so (the HIP/gfx950 C-ABI library) in-tree with hipcc.

Every .hip source under csrc/ is compiled to its own object (in parallel) and the
objects are linked into quantized_sparse_moe_amd/libqsmoe.so.  Objects live in
_build/ (git-ignored).  Run:  python -m quantized_sparse_moe_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "qsmoe")
LIB = os.path.join(HERE, "libqsmoe.so")
ARCH = os.environ.get("QSMOE_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    r = subprocess.run(["hipcc", *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    noise = ("not a recognized feature", "argument unused during compilation")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
