"""Build libmoe_mxfp4.so for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mxfp4.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["status.cpp", "pack.hip", "quant.hip", "route.hip", "ffn.hip", "stream.hip",
           "prefill.hip", "down_rows.hip", "router.hip"]
# Packed-fp32 VALU ops are disabled: only scalar fp32 FMAs are emitted.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_library(jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    _build_counters()
    return LIB


COUNTERS = os.path.join(HERE, "moe_counters")


def _build_counters() -> None:
    """The native counters driver (tools/moe_counters.cpp), linked to the library."""
    src = os.path.join(HERE, "tools", "moe_counters.cpp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-I", os.path.join(os.path.dirname(HERE), "include"), src, "-L", HERE,
           "-lmoe_mxfp4", "-Wl,-rpath,$ORIGIN", "-o", COUNTERS + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for moe_counters:\n{r.stderr}")
    os.replace(COUNTERS + ".tmp", COUNTERS)


if __name__ == "__main__":
    print(build_library())
