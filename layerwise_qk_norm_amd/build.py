"""Build libqknorm.so for gfx950 with hipcc (in-tree, no JIT cache)."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqknorm.so")
ROOT = os.path.dirname(PKG)

# (source, extra flags, object name); the row kernels are compiled once per storage pair
UNITS = [
    ("api.cpp", [], "api"),
    ("rows.hip", [], "rows"),
    ("rows_inst.hip", ["-DQKN_ROWS_BF=1", "-DQKN_ROWS_GBF=1"], "rows_bf16_gbf16"),
    ("rows_inst.hip", ["-DQKN_ROWS_BF=1", "-DQKN_ROWS_GBF=0"], "rows_bf16_gf32"),
    ("rows_inst.hip", ["-DQKN_ROWS_BF=0", "-DQKN_ROWS_GBF=1"], "rows_f32_gbf16"),
    ("rows_inst.hip", ["-DQKN_ROWS_BF=0", "-DQKN_ROWS_GBF=0"], "rows_f32_gf32"),
    ("gemm.hip", [], "gemm"),
    ("shard.hip", [], "shard"),
]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(unit) -> str:
    src, extra, name = unit
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), *CFLAGS, *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libqknorm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    workers = max(1, min(len(UNITS), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
