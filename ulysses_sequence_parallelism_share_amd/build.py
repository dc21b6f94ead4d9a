"""Build libulysses_sp.so (gfx950 only) in-tree with hipcc.

    python -m ulysses_sequence_parallelism_share_amd.build

Objects go to <repo>/_build/, the shared library next to this file.  Every
call recompiles (the build is a few seconds per file, run in parallel).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libulysses_sp.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result", "-fvisibility=hidden",
    # the compiler must not form packed fp32 VALU instructions; fp32 math stays scalar
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Machine-scheduler strategy per source (LLVM AMDGPU option), measured on the
# 500K-token rank share against the default strategy in alternating runs:
# the forward 2.4 % faster with iterative-ilp, the dK/dV kernel 1.3 % faster
# with max-ilp (dQ unchanged); other sources keep the default.
PER_SOURCE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *PER_SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
