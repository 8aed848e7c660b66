"""ctypes binding of libpkv_probe.so: the read-only bandwidth probe
(include/pkv_probe.h), used by bench.py to measure the HBM rate of the split
kernel's own access pattern.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

from . import _lib  # loads torch's HIP runtime before the probe library

PROBE_LIB_PATH = os.path.join(_lib.PKG_DIR, "libpkv_probe.so")
EXPORTED = ("pkv_probe_read", "pkv_probe_read_lds", "pkv_probe_stream", "pkv_probe_empty",
            "pkv_probe_sleep")
LDS_SHAPES = ((4, 2), (4, 4), (8, 2), (2, 7))  # (waves, pages in LDS per wave)

if not os.path.exists(PROBE_LIB_PATH):
    raise ImportError(f"{PROBE_LIB_PATH} is not built; run python -m paged_kv_gqa_block_amd.build")
LIB = ctypes.CDLL(PROBE_LIB_PATH)
LIB.pkv_probe_read.restype = ctypes.c_int
LIB.pkv_probe_read.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4
LIB.pkv_probe_read_lds.restype = ctypes.c_int
LIB.pkv_probe_read_lds.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int32] * 3 +
                                   [ctypes.c_void_p] * 2 + [ctypes.c_int32] * 3 +
                                   [ctypes.c_void_p] * 2)
LIB.pkv_probe_stream.restype = ctypes.c_int
LIB.pkv_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p]
LIB.pkv_probe_empty.restype = ctypes.c_int
LIB.pkv_probe_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
LIB.pkv_probe_sleep.restype = ctypes.c_int
LIB.pkv_probe_sleep.argtypes = [ctypes.c_int32, ctypes.c_void_p]


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


def _stream_ptr(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def probe_read_lds(w: dict, step, waves: int, depth: int, consume: bool, sink: torch.Tensor,
                   stream=None) -> None:
    """The same pages through LDS rings of `depth` pages per wave (head_dim 128)."""
    n = max(1, int(step.info.n_tasks)) * waves * 64
    if sink.numel() < n or sink.dtype != torch.int32:
        raise ValueError("sink must hold n_tasks * waves * 64 int32")
    rc = LIB.pkv_probe_read_lds(w["k_pool"].data_ptr(), w["v_pool"].data_ptr(),
                                w["block_table"].data_ptr(), w["block_table"].shape[1],
                                step.prob.num_kv_heads, step.prob.head_dim,
                                step.plan_host.data_ptr(), step.plan_dev.data_ptr(), waves, depth,
                                int(consume), sink.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_read_lds failed ({rc})")


def probe_stream(buf: torch.Tensor, nbytes: int, grid: int, loads_in_flight: int,
                 sink: torch.Tensor, stream=None) -> None:
    """Contiguous read of the first `nbytes` bytes of `buf`."""
    if nbytes > buf.numel() * buf.element_size() or sink.numel() < grid:
        raise ValueError("buffer or sink too small")
    rc = LIB.pkv_probe_stream(buf.data_ptr(), nbytes, grid, loads_in_flight, sink.data_ptr(),
                              _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_stream failed ({rc})")


def probe_empty(grid: int, threads: int, flag=None, stream=None) -> None:
    """A launch of `grid` x `threads` that does (almost) nothing."""
    if flag is not None and (flag.numel() < 2 or flag.dtype != torch.int32):
        raise ValueError("flag must hold two int32")
    rc = LIB.pkv_probe_empty(grid, threads, None if flag is None else flag.data_ptr(),
                             _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_empty failed ({rc})")


def probe_sleep(microseconds: int, stream=None) -> None:
    """Keep the device busy for `microseconds` (enqueued before a timed window)."""
    rc = LIB.pkv_probe_sleep(int(microseconds), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"pkv_probe_sleep failed ({rc})")
