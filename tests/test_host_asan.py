"""Host code of libtq under AddressSanitizer (CPU only).

The library is built a second time with its host pass instrumented (argument
checks, launch set-up, the fp64 codebook solver), and every ABI test runs
against that copy in a child process that preloads the ASan runtime.  No call
reaches the GPU: the ABI tests stop at the argument checks or stay in host
code.  A heap or stack overrun in the host code aborts the child with an ASan
report, which fails this test."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "embedding_vector_quantization_amd", "csrc"))
import build as libbuild  # noqa: E402


@pytest.mark.skipif(not os.path.exists(libbuild.HIPCC), reason="hipcc not available")
def test_abi_suite_clean_under_host_asan():
    lib = libbuild.build_asan(verbose=False)
    runtime = libbuild.asan_runtime()
    env = dict(os.environ)
    env.update(TQ_ABI_LIB=lib, LD_PRELOAD=runtime,
               # the interpreter itself is not instrumented and keeps its
               # allocations to the end; leaks are not what this checks
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_abi.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert re.search(r"\b\d+ passed\b", out) and not re.search(r"\b\d+ skipped\b", out), out[-2000:]
