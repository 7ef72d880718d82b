"""Build libmiattn.so (gfx950 only) in-tree with hipcc.

    python -m exact_tiled_attention_13_amd.build [--sanitize]

Compiles every source under csrc/ to an object in parallel and links one
shared library next to this file.  hipcc cross-compiles for gfx950 without a
GPU present.

``--sanitize`` builds instead ``_build/san/libmiattn_san.so``: the host code
of every source (the C ABI layer, the launch table, the launchers) under
AddressSanitizer and UndefinedBehaviorSanitizer, the device code as usual,
for running the CPU tests of the ABI and the launch table against it
(``tests/test_sanitizer.py``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmiattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "tiles.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip", "noalloc.hip"]

# Per-file flags.  The bf16 prefill kernel never lets NaN reach its softmax
# (rows past a sequence's length are replaced by finite rows before the
# math), so it may drop the NaN quieting that IEEE max would otherwise need.
FILE_FLAGS = {"fwd_bf16.hip": ["-fno-honor-nans"]}

COMMON_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed-fp32 VALU instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


# Host-only sanitizers: every -fsanitize= applies to the host pass only
# (each preceded by -Xarch_host); the device code is not instrumented.
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libmiattn_san.so")


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; ROCm is required to build libmiattn.so")
    return h


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SAN_DIR if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    extra = [*SAN_FLAGS, "-g"] if sanitize else []
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libmiattn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmiattn.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """Host-only ASan/UBSan build of every source; returns the library path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize=True), SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", *SAN_FLAGS, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {SAN_LIB} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
