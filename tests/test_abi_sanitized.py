"""The host side of the library (argument validation, workspace planning,
frame tables, the no-alloc size check) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: tests/test_abi.py runs in a child
process against the host-sanitized build (build_lib.build(sanitize=True))
with the ASan runtime preloaded, and must finish without a report.  A
planted out-of-bounds write (frame tables into arrays one frame too short)
shows the sanitizer is live in that set-up."""
import os
import subprocess
import sys

import pytest

from hybrid_softmax_linear_block_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env():
    if not os.path.exists(build_lib.SAN_LIB):
        build_lib.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=build_lib.asan_runtime(), HYB_ATTN_LIB=build_lib.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    return env


def test_abi_checks_pass_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], env=_env(), cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]


PLANTED = r"""
import ctypes, numpy as np
from hybrid_softmax_linear_block_amd import api
lib = api.load()
assert api.LIB_PATH.endswith("san/libhybattn.so"), api.LIB_PATH
lay = api.Layout(1, 6, 1, 0, 1, 64).c()
short = [np.zeros(n, np.int32) for n in (5 * 5, 5, 5 * 2, 5 * 2)]   # sized for 5 frames, not 6
ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
lib.hyb_layout_tables(ctypes.byref(lay), *[ptr(a) for a in short])
print("no report")
"""


def test_sanitizer_catches_a_planted_overflow():
    r = subprocess.run([sys.executable, "-c", PLANTED], env=_env(), cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.returncode, r.stdout, r.stderr[-2000:])
