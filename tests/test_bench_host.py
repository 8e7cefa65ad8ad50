"""Host-side logic of bench.py (no GPU): the kernel-source hash that keys the
committed rocprofv3 counter summary ignores comments and layout but not code."""

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_code_only_drops_comments_keeps_literals():
    src = ('int a = 1;   // a comment\n/* block\n   comment */ const char *s = "x // y /* z */";\n'
           "char c = '/'; int q = r / t;\n")
    assert bench._code_only(src) == 'int a = 1; const char *s = "x // y /* z */"; char c = \'/\'; int q = r / t;'


def test_code_only_sees_code_changes():
    a = "__global__ void k(float *p) { p[0] = 1.0f; }  // first\n"
    b = "__global__ void k(float *p) {\n  p[0] = 1.0f;   /* reworded */\n}\n"
    c = "__global__ void k(float *p) { p[0] = 2.0f; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_source_hash_is_stable():
    assert bench.source_hash() == bench.source_hash()
    assert len(bench.source_hash()) == 16
