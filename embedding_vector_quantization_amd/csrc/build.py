"""Builds libtq.so (the TurboQuant HIP library) in-tree for gfx950, and
libtqprobe.so (HBM bandwidth probes the benchmark uses for reference rates).

Usage: python embedding_vector_quantization_amd/csrc/build.py [--jobs N] [--asan]

Every source is compiled on every call (object files go to _build/ at the
repository root); the shared libraries land next to the Python binding.

--asan builds a second copy of libtq, _build/asan/libtq_asan.so, whose host
code (argument checks, launch set-up, the codebook solver) is instrumented by
AddressSanitizer; the device code is the same.  It is a CPU-side check only:
load it into a process that preloads the ASan runtime (asan_runtime() names
it) and call the host paths.
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
PROBE_LIB = os.path.join(PKG, "libtqprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["tq_api.cpp", "tq_codebook.cpp", "tq_encode.hip", "tq_decode.hip", "tq_score.hip", "tq_scorem.hip", "tq_attend.hip", "tq_topk.hip"]
PROBE_SOURCES = ["tq_probe.hip"]
# the issue probe's MFMA accumulators stay in ordinary VGPRs, so its loops
# hold no accumulator-register moves
EXTRA = {"tq_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libtq_asan.so")
# AddressSanitizer for the host pass only (device code is not instrumented)
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _compile(src: str, out_dir: str = BUILD, extra: tuple = ()) -> tuple[str, float, str]:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *extra, "-c", os.path.join(HERE, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"] if src == "tq_api.cpp" else []
    t0 = time.time()
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    noise = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, time.time() - t0, noise


def _link(objs, lib, extra: tuple = ()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", *extra, "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    every = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(every), os.cpu_count() or 4)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, every))
    objs = {}
    for (obj, dt, noise), src in zip(results, every):
        objs[src] = obj
        if verbose:
            print(f"  {src:18s} {dt:6.1f} s", flush=True)
            if noise.strip():
                print(noise, flush=True)
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB} in {time.time() - t0:.1f} s", flush=True)
    return LIB


def build_asan(jobs: int | None = None, verbose: bool = True) -> str:
    """libtq with AddressSanitizer in its host code, at ASAN_LIB."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, ASAN_DIR, tuple(ASAN_HOST)), SOURCES))
    _link([obj for obj, _, _ in results], ASAN_LIB, tuple(ASAN_HOST))
    if verbose:
        print(f"built {ASAN_LIB} in {time.time() - t0:.1f} s", flush=True)
    return ASAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into a process
    that loads ASAN_LIB)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm")
    if not os.path.isdir(llvm):
        llvm = "/opt/rocm/llvm"
    proc = subprocess.run([os.path.join(llvm, "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True)
    path = proc.stdout.strip()
    if proc.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
        if not hits:
            raise RuntimeError("the compiler's shared ASan runtime was not found")
        path = hits[-1]
    return os.path.realpath(path)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--asan", action="store_true", help="build the host-ASan copy of libtq instead")
    args = ap.parse_args()
    try:
        build_asan(args.jobs) if args.asan else build(args.jobs)
    except RuntimeError as exc:
        print(exc, file=sys.stderr)
        sys.exit(1)
