"""Build libawq_mi355x.so (gfx950) in-tree with hipcc.

    python -m weight_only_int4_awq_amd.build      # or build() from Python

Every source is compiled for gfx950 only, without fast-math (the kernels rely
on IEEE division, fp16/fp32/fp64 denormals and unfused multiply-adds unless
written as fma), and with packed fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libawq_mi355x.so"
SOURCES = ("api.hip", "calib_stats.hip", "search.hip", "pack.hip", "linear.hip", "linear_wbit.hip", "mixed.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-I", str(ROOT / "include"),
]


def _compile(src: pathlib.Path, obj: pathlib.Path) -> None:
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every HIP source and link the shared library; returns its path."""
    if not pathlib.Path(HIPCC).exists() and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    BUILD.mkdir(exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = []
        for s in SOURCES:
            obj = BUILD / (s.replace(".hip", ".o"))
            objs.append(obj)
            futs.append(ex.submit(_compile, CSRC / s, obj))
        for f in futs:
            f.result()
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
