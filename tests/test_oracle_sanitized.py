"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle takes raw pointers and sizes from ctypes.  Here the same source is
built with -fsanitize=address,undefined (host code, gcc) and the oracle's pin
suite runs against that build in a child process with the sanitizer runtimes
preloaded: any out-of-bounds access, use of freed memory, signed overflow,
bad shift or misaligned access in the oracle ends the run with a report.  A
canary first shows that the instrumentation is live (a deliberately short
output buffer is reported)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_packing.py", "test_oracle_formats.py", "test_oracle_dequant.py",
             "test_oracle_linear.py", "test_oracle_swiglu.py", "test_oracle_hadamard.py"]


def runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def san_env():
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update({"LD_PRELOAD": f"{asan}:{ubsan}", "WQ_ORACLE_LIB": lib,
                "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "PYTHONPATH": ROOT})
    return env


def test_sanitizer_is_live(san_env):
    # 4-bit codes of a 64 x 8 layer unpack into K*N = 512 bytes; give 511
    code = ("import numpy as np, oracle; L = oracle.lib(); "
            "import ctypes; q = np.zeros((8, 8), np.uint32); out = np.zeros(511, np.uint8); "
            "maps = open('/proc/self/maps').read(); assert 'liboracle_san.so' in maps; "
            "L.wqo_unpack_codes(q.ctypes.data, 64, 8, 4, out.ctypes.data)")
    r = subprocess.run([sys.executable, "-c", code], env=san_env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_pins_clean_under_sanitizers(san_env):
    files = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                       env=san_env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in r.stdout
