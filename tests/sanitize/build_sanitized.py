"""Build libpkv's host code with AddressSanitizer and UndefinedBehaviorSanitizer.

    python tests/sanitize/build_sanitized.py   -> tests/sanitize/_build/libpkv_san.so

The host translation units (planner.cpp, cost_model.cpp, api.cpp,
noalloc_api.cpp) are compiled with g++ and linked with stub kernel launchers
and a stub scratch-address lookup (stub_launchers.cpp)
against the HIP runtime; no device code is built.  Load the result through
the binding by setting PKV_LIBRARY to its path and preloading the ASan
runtime (see tests/test_sanitized_host.py).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "paged_kv_gqa_block_amd", "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libpkv_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = [os.path.join(CSRC, f) for f in ("planner.cpp", "cost_model.cpp", "api.cpp",
                                                   "noalloc_api.cpp")] + \
    [os.path.join(HERE, "stub_launchers.cpp")]
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
         f"-I{CSRC}"]


def asan_runtime() -> str:
    """Path of g++'s ASan runtime, to preload into the Python process."""
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", *FLAGS, *SOURCES, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitizer build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
