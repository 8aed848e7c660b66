"""ctypes binding of libpkv_probe.so: the read-only bandwidth probe
(include/pkv_probe.h), used by bench.py to measure the HBM rate of the split
kernel's own access pattern.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

from . import _lib  # loads torch's HIP runtime before the probe library

PROBE_LIB_PATH = os.path.join(_lib.PKG_DIR, "libpkv_probe.so")
EXPORTED = ("pkv_probe_read",)

if not os.path.exists(PROBE_LIB_PATH):
    raise ImportError(f"{PROBE_LIB_PATH} is not built; run python -m paged_kv_gqa_block_amd.build")
LIB = ctypes.CDLL(PROBE_LIB_PATH)
LIB.pkv_probe_read.restype = ctypes.c_int
LIB.pkv_probe_read.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4


def probe_read(w: dict, step, sink: torch.Tensor, stream=None) -> None:
    """Read every page chunk of `step`'s plan tasks from w's pools."""
    hkv = step.prob.num_kv_heads
    d = step.prob.head_dim
    if sink.numel() < max(1, int(step.info.n_tasks)) or sink.dtype != torch.int32:
        raise ValueError("sink must hold one int32 per task")
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = LIB.pkv_probe_read(w["k_pool"].data_ptr(), w["v_pool"].data_ptr(),
                            w["block_table"].data_ptr(), w["block_table"].shape[1], hkv, d,
                            step.plan_host.data_ptr(), step.plan_dev.data_ptr(),
                            sink.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_read failed ({rc})")
