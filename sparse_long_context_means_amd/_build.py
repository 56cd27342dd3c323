"""Compiles the HIP library (libmpattn.so) for gfx950 in-tree."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmpattn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "kmeans.hip", "codes.hip", "decode.hip", "unit.hip", "hier.hip", "dense.hip", "probe.hip"]
ARCH = os.environ.get("MPATTN_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU forms stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source additions: the k-means assignment keeps its matrix-core
# accumulators in ordinary vector registers, which its argmax reads directly
# (no copies out of the accumulator registers)
EXTRA_FLAGS = {"kmeans.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def flags_for(src: str) -> list:
    return [*FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), [])]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
