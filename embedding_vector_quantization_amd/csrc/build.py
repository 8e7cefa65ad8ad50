"""Builds libtq.so (the TurboQuant HIP library) in-tree for gfx950.

Usage: python embedding_vector_quantization_amd/csrc/build.py [--jobs N]

Every source is compiled on every call (object files go to _build/ at the
repository root); the shared library lands next to the Python binding.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["tq_api.cpp", "tq_codebook.cpp", "tq_encode.hip", "tq_decode.hip", "tq_score.hip", "tq_scorem.hip", "tq_attend.hip", "tq_topk.hip"]

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src: str) -> tuple[str, float, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(HERE, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"] if src == "tq_api.cpp" else []
    t0 = time.time()
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    noise = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, time.time() - t0, noise


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for (obj, dt, noise), src in zip(results, SOURCES):
        objs.append(obj)
        if verbose:
            print(f"  {src:18s} {dt:6.1f} s", flush=True)
            if noise.strip():
                print(noise, flush=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", flush=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as exc:
        print(exc, file=sys.stderr)
        sys.exit(1)
