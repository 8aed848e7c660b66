"""Compile libpkv.so (host planner + HIP kernels for gfx950) and the
read-bandwidth probe libpkv_probe.so (a measurement tool) in-tree.

    python -m paged_kv_gqa_block_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libpkv.so")
PROBE_LIB_PATH = os.path.join(PKG, "libpkv_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [
    "planner.cpp", "api.cpp", "merge.hip", "split_valu.hip", "split_mfma.hip", "planner_device.hip",
    "append.hip", "cost_model.cpp", "noalloc.hip", "noalloc_api.cpp",
]
PROBE_SOURCES = ["read_probe.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Wall", "-Wno-unused-result",
]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source additions.  merge.hip: the leading scalar kernel parameters
# (14 dwords) are preloaded into SGPRs at wave launch.
EXTRA_FLAGS = {"merge.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=14"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, [])]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
