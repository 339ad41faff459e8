"""The CPU tests of the C ABI (tests/test_abi_host.py) again, against the AddressSanitizer build
of the library's host code (libattn_asan.so) with the sanitizer runtime preloaded: argument
validation, workspace sizing and the host block table must make no out-of-bounds access, use
after free or other memory error that ASan detects.  Runs in a child process; no GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_LIB = os.path.join(ROOT, "exact_io_aware_21_amd", "libattn_asan.so")


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_tests_under_asan():
    rt = asan_runtime()
    if rt is None or not os.path.exists(ASAN_LIB):
        pytest.fail("the ASan runtime or libattn_asan.so is missing (make -C "
                    "exact_io_aware_21_amd/csrc)")
    env = dict(os.environ, LD_PRELOAD=rt, ATTN_LIB_PATH=ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert r.returncode == 0


PROBE = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
from exact_io_aware_21_amd import attn
L = attn.lib()
maps = open("/proc/self/maps").read()
assert "libclang_rt.asan" in maps and "libattn_asan.so" in maps, "not the sanitized build"
# a caller bug: a kv_list buffer one element short of n_qt * n_kt (host block table)
N, d = 300, 64
n_qt, n_kt = 2, 5
cls = np.zeros(n_qt * n_kt, np.int8)
cnt = np.zeros(n_qt, np.int32)
lst = np.zeros(n_qt * n_kt - 1, np.int32)
p = attn.attn_params()
print("calling", flush=True)
L.attn_block_table_host(1, 1, N, d, attn.ATTN_MASK_CAUSAL, ctypes.byref(p),
                                 cls.ctypes.data, cnt.ctypes.data, lst.ctypes.data)
print("no report", flush=True)
"""


def test_asan_is_live_in_the_library():
    """The sanitized library reports a write past a caller's undersized host buffer (a caller
    bug the C ABI cannot see), which shows that the checks above ran with ASan active."""
    rt = asan_runtime()
    if rt is None or not os.path.exists(ASAN_LIB):
        pytest.fail("the ASan runtime or libattn_asan.so is missing")
    env = dict(os.environ, LD_PRELOAD=rt, ATTN_LIB_PATH=ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=86")
    r = subprocess.run([sys.executable, "-c", PROBE, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    assert "calling" in r.stdout and "no report" not in r.stdout, r.stdout + r.stderr[-2000:]
    assert r.returncode == 86
    assert "heap-buffer-overflow" in r.stderr and "attn_block_table_host" in r.stderr
