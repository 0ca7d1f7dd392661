"""Build librudder.so (HIP, gfx950) in-tree with hipcc.

Every translation unit under csrc/ is compiled for gfx950 only, with fp
contraction off (the epilogue's single fma is explicit) and packed-fp32
instruction selection disabled, then linked into one shared library next to
this file (_lib/librudder.so).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
GEN_DIR = os.path.join(BUILD_DIR, "gen")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "librudder.so")
ARCH = os.environ.get("RUDDER_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}", f"-I{GEN_DIR}",
]


def generate_tables() -> None:
    """Build-time tables: the GELU table (csrc/gelu_table_gen.cpp, a host
    program) is written to _build/gen/gelu_table.inc for w4_gemm.hip."""
    os.makedirs(GEN_DIR, exist_ok=True)
    exe = os.path.join(BUILD_DIR, "gelu_table_gen")
    src = os.path.join(CSRC, "gelu_table_gen.cpp")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", src, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for {src}:\n{r.stdout}\n{r.stderr}")
    out = os.path.join(GEN_DIR, "gelu_table.inc")
    r = subprocess.run([exe, out + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{exe} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    generate_tables()
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
