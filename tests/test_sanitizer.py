"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

`python -m exact_tiled_attention_13_amd.build --sanitize` (also run by
`__graft_entry__.build()`) builds `_build/san/libmiattn_san.so`: the host
code of every source instrumented (address errors, undefined behaviour,
which aborts), the device code as usual.  This test runs the CPU tests of
the ABI (argument checks, error codes, exported symbols, the binding's
checks) and of the launch table (lookups, JSON, concurrent set/lookup)
against that library in a child process with the sanitizer runtime
preloaded, and requires a clean run.  Leak checking is off: the Python
interpreter itself is not instrumented and keeps memory until exit.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "exact_tiled_attention_13_amd", "_build", "san", "libmiattn_san.so")


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_and_tile_table_clean_under_sanitizers():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime under /opt/rocm/llvm")
    if not os.path.exists(SAN_LIB):
        pytest.skip("sanitized library not built (python -m exact_tiled_attention_13_amd.build --sanitize)")
    env = dict(os.environ)
    env.update(MIATTN_LIB=SAN_LIB, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    # the child loads the sanitized library, not the regular one
    probe = subprocess.run([sys.executable, "-c", "from exact_tiled_attention_13_amd import _lib; _lib.load(); "
                            "print(_lib.LIB_PATH)"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip().endswith("libmiattn_san.so")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_tiles.py", "-m", "not gpu",
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out
