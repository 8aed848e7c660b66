"""ctypes binding of libpkv.so (include/pkv.h).

Argument marshalling only: every step of the decode path runs in the
library's host planner and HIP kernels.  torch tensors are accepted wherever
the C ABI takes a pointer (their ``data_ptr()`` is passed); numpy arrays are
accepted for host buffers.  A missing or stale library raises at import of
this module -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# torch ships its own HIP runtime (libamdhip64, soname libamdhip64.so.7).  It
# must be the one libpkv binds to: importing torch first makes the dynamic
# loader resolve libpkv's libamdhip64.so.7 to torch's already-loaded copy, so
# device pointers and streams from torch are valid inside the library.  If
# libpkv were loaded first, torch would load a second runtime.
import torch  # noqa: F401  (load order matters, see above)

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library (for instance the
# sanitizer build of its host code that the CPU tests load); the default is
# the in-tree libpkv.so.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(PKG_DIR, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ESHAPE, PKV_EDTYPE, PKV_ERANGE, PKV_ENOSPC, PKV_EHIP = 0, -1, -2, -3, -4, -5, -6
PKV_F16, PKV_BF16 = 0, 1
PKV_BUCKETED, PKV_WORKQUEUE, PKV_NOSPLIT, PKV_PADDED = 0, 1, 2, 3
PKV_KERNEL_AUTO, PKV_KERNEL_VALU, PKV_KERNEL_MFMA = 0, 1, 2
PKV_PLAN_MAGIC = 0x31564B50
PKV_PLAN_HEADER_WORDS = 16

PATH_NAMES = {PKV_BUCKETED: "bucketed", PKV_WORKQUEUE: "workqueue", PKV_NOSPLIT: "nosplit",
              PKV_PADDED: "padded"}
PATH_IDS = {v: k for k, v in PATH_NAMES.items()}
DTYPE_IDS = {"f16": PKV_F16, "bf16": PKV_BF16}
KERNEL_IDS = {"auto": PKV_KERNEL_AUTO, "valu": PKV_KERNEL_VALU, "mfma": PKV_KERNEL_MFMA}

EXPORTED = ("pkv_plan_bytes", "pkv_plan", "pkv_plan_get_info", "pkv_decode", "pkv_merge",
            "pkv_plan_device", "pkv_decode_device", "pkv_merge_device", "pkv_decode_selfplan",
            "pkv_merge_selfplan", "pkv_append_kv",
            "pkv_policy", "pkv_cost_features", "pkv_policy_model", "pkv_policy_default",
            "pkv_balanced_splits",
            "pkv_noalloc_bytes", "pkv_attend_noalloc", "pkv_status_str")
PKV_COST_FEATURES = 8


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class pkv_problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int32),
        ("max_pages_per_row", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("kernel", ctypes.c_int32),
    ]


class pkv_plan_info(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("n_tasks", ctypes.c_int32),
        ("n_buckets", ctypes.c_int32),
        ("n_launches", ctypes.c_int32),
        ("n_state_slots", ctypes.c_int32),
        ("n_empty_slots", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("kv_bytes", ctypes.c_int64),
        ("merge_state_bytes", ctypes.c_int64),
        ("plan_bytes", ctypes.c_int64),
        ("max_task_pages", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class pkv_policy_table(ctypes.Structure):
    _fields_ = [("n_rules", ctypes.c_int32), ("rules", ctypes.POINTER(ctypes.c_int32))]


class pkv_cost_model(ctypes.Structure):
    _fields_ = [("n_candidates", ctypes.c_int32), ("candidates", ctypes.POINTER(ctypes.c_int32)),
                ("weights", ctypes.POINTER(ctypes.c_float)), ("num_cus", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_gqa_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_hip_runtime()
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_float)
    prob_p = ctypes.POINTER(pkv_problem)
    lib.pkv_plan_bytes.argtypes = [prob_p, i32, i32]
    lib.pkv_plan_bytes.restype = ctypes.c_size_t
    lib.pkv_plan.argtypes = [prob_p, vp, i32, i32, vp, vp, ctypes.c_size_t,
                             ctypes.POINTER(pkv_plan_info), vp]
    lib.pkv_plan.restype = i32
    lib.pkv_plan_get_info.argtypes = [prob_p, vp, ctypes.POINTER(pkv_plan_info)]
    lib.pkv_plan_get_info.restype = i32
    lib.pkv_decode.argtypes = [prob_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_decode.restype = i32
    lib.pkv_merge.argtypes = [prob_p, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_merge.restype = i32
    lib.pkv_plan_device.argtypes = [prob_p, vp, i32, vp, ctypes.c_size_t, vp, vp]
    lib.pkv_plan_device.restype = i32
    lib.pkv_decode_device.argtypes = [prob_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_decode_device.restype = i32
    lib.pkv_merge_device.argtypes = [prob_p, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_merge_device.restype = i32
    lib.pkv_decode_selfplan.argtypes = [prob_p, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_decode_selfplan.restype = i32
    lib.pkv_merge_selfplan.argtypes = [prob_p, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_merge_selfplan.restype = i32
    lib.pkv_append_kv.argtypes = [prob_p, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_append_kv.restype = i32
    lib.pkv_policy.argtypes = [ctypes.POINTER(pkv_policy_table), i32, i32,
                               ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.pkv_policy.restype = i32
    lib.pkv_cost_features.argtypes = [prob_p, vp, i32, i32, i32, vp, vp]
    lib.pkv_cost_features.restype = i32
    lib.pkv_policy_model.argtypes = [prob_p, ctypes.POINTER(pkv_cost_model), vp, vp,
                                     ctypes.POINTER(i32), ctypes.POINTER(i32), f32p]
    lib.pkv_policy_model.restype = i32
    lib.pkv_policy_default.argtypes = [ctypes.POINTER(pkv_policy_table),
                                       ctypes.POINTER(pkv_cost_model), prob_p, vp, vp,
                                       ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.pkv_policy_default.restype = i32
    lib.pkv_balanced_splits.argtypes = [prob_p, vp, i32, i32, i32, ctypes.POINTER(i32)]
    lib.pkv_balanced_splits.restype = i32
    lib.pkv_noalloc_bytes.argtypes = [prob_p, i32]
    lib.pkv_noalloc_bytes.restype = ctypes.c_size_t
    lib.pkv_attend_noalloc.argtypes = [prob_p, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.pkv_attend_noalloc.restype = i32
    lib.pkv_status_str.argtypes = [i32]
    lib.pkv_status_str.restype = ctypes.c_char_p
    return lib


def _check_single_hip_runtime() -> None:
    """Fail loudly if two different libamdhip64 copies are mapped."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:  # pragma: no cover
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError(f"two HIP runtimes loaded: {sorted(real)}")


LIB = _load()


def pkv_status_str(status: int) -> str:
    return LIB.pkv_status_str(status).decode()


def _check(fn: str, status: int) -> None:
    if status != PKV_OK:
        raise PkvError(fn, status, pkv_status_str(status))


def _ptr(x) -> int | None:
    """Address of a torch tensor / numpy array / raw int; None stays NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    assert x.is_contiguous(), "tensors passed to libpkv must be contiguous"
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_problem(batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pool_pages,
                 max_pages_per_row, dtype="f16", sm_scale=None, kernel="auto") -> pkv_problem:
    if sm_scale is None:
        sm_scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    return pkv_problem(batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pool_pages,
                       max_pages_per_row, DTYPE_IDS.get(dtype, dtype) if isinstance(dtype, str)
                       else dtype, sm_scale, KERNEL_IDS[kernel] if isinstance(kernel, str)
                       else kernel)


def pkv_plan_bytes(prob: pkv_problem, path: int, max_splits: int) -> int:
    return LIB.pkv_plan_bytes(ctypes.byref(prob), path, max_splits)


def pkv_plan(prob: pkv_problem, seq_lens_host, path: int, max_splits: int, plan_host,
             plan_dev=None, plan_bytes: int | None = None, stream=None) -> pkv_plan_info:
    info = pkv_plan_info()
    if plan_bytes is None:
        plan_bytes = plan_host.numel() * plan_host.element_size() if hasattr(
            plan_host, "numel") else plan_host.nbytes
    seq = seq_lens_host
    if isinstance(seq, np.ndarray):
        assert seq.dtype == np.int32 and seq.flags["C_CONTIGUOUS"]
    else:
        assert str(seq.dtype) == "torch.int32" and seq.device.type == "cpu"
    _check("pkv_plan", LIB.pkv_plan(ctypes.byref(prob), _ptr(seq), path, max_splits,
                                    _ptr(plan_host), _ptr(plan_dev), plan_bytes,
                                    ctypes.byref(info), _stream(stream)))
    return info


def bind_call(fn: str, *args) -> tuple:
    """Marshal the arguments of one C entry point once: (fn, converted args).
    ``call_bound`` then makes the call with no per-call conversion, which keeps
    the host's launch rate above the device's for steps of ~10 µs."""
    conv = tuple(ctypes.byref(a) if isinstance(a, ctypes.Structure) else
                 (_stream(a) if isinstance(a, torch.cuda.Stream) else _ptr(a)) for a in args)
    return fn, getattr(LIB, fn), conv


def call_bound(bound: tuple) -> None:
    fn, f, args = bound
    status = f(*args)
    if status != PKV_OK:
        _check(fn, status)


def pkv_plan_get_info(prob: pkv_problem, plan_host) -> pkv_plan_info:
    info = pkv_plan_info()
    _check("pkv_plan_get_info",
           LIB.pkv_plan_get_info(ctypes.byref(prob), _ptr(plan_host), ctypes.byref(info)))
    return info


def pkv_decode(prob: pkv_problem, plan_host, plan_dev, q, k_pool, v_pool, block_table,
               seq_lens_dev, st_m=None, st_l=None, st_o=None, out=None, lse=None,
               stream=None) -> None:
    _check("pkv_decode", LIB.pkv_decode(
        ctypes.byref(prob), _ptr(plan_host), _ptr(plan_dev), _ptr(q), _ptr(k_pool),
        _ptr(v_pool), _ptr(block_table), _ptr(seq_lens_dev), _ptr(st_m), _ptr(st_l),
        _ptr(st_o), _ptr(out), _ptr(lse), _stream(stream)))


def pkv_merge(prob: pkv_problem, plan_host, plan_dev, st_m, st_l, st_o, out, lse=None,
              stream=None) -> None:
    _check("pkv_merge", LIB.pkv_merge(
        ctypes.byref(prob), _ptr(plan_host), _ptr(plan_dev), _ptr(st_m), _ptr(st_l),
        _ptr(st_o), _ptr(out), _ptr(lse), _stream(stream)))


def pkv_plan_device(prob: pkv_problem, seq_lens_dev, max_splits: int, plan_dev,
                    plan_bytes: int | None = None, bad_rows_dev=None, stream=None) -> None:
    if plan_bytes is None:
        plan_bytes = plan_dev.numel() * plan_dev.element_size()
    _check("pkv_plan_device", LIB.pkv_plan_device(
        ctypes.byref(prob), _ptr(seq_lens_dev), max_splits, _ptr(plan_dev), plan_bytes,
        _ptr(bad_rows_dev), _stream(stream)))


def pkv_decode_device(prob: pkv_problem, plan_dev, max_splits: int, q, k_pool, v_pool,
                      block_table, st_m, st_l, st_o, stream=None) -> None:
    _check("pkv_decode_device", LIB.pkv_decode_device(
        ctypes.byref(prob), _ptr(plan_dev), max_splits, _ptr(q), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(st_m), _ptr(st_l), _ptr(st_o), _stream(stream)))


def pkv_merge_device(prob: pkv_problem, plan_dev, st_m, st_l, st_o, out, lse=None,
                     stream=None) -> None:
    _check("pkv_merge_device", LIB.pkv_merge_device(
        ctypes.byref(prob), _ptr(plan_dev), _ptr(st_m), _ptr(st_l), _ptr(st_o), _ptr(out),
        _ptr(lse), _stream(stream)))


def pkv_decode_selfplan(prob: pkv_problem, seq_lens_dev, max_splits: int, work_counter_dev, q,
                        k_pool, v_pool, block_table, st_m, st_l, st_o, stream=None) -> None:
    _check("pkv_decode_selfplan", LIB.pkv_decode_selfplan(
        ctypes.byref(prob), _ptr(seq_lens_dev), max_splits, _ptr(work_counter_dev), _ptr(q),
        _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(st_m), _ptr(st_l), _ptr(st_o),
        _stream(stream)))


def pkv_merge_selfplan(prob: pkv_problem, seq_lens_dev, max_splits: int, work_counter_dev, st_m,
                       st_l, st_o, out, lse=None, stream=None) -> None:
    _check("pkv_merge_selfplan", LIB.pkv_merge_selfplan(
        ctypes.byref(prob), _ptr(seq_lens_dev), max_splits, _ptr(work_counter_dev), _ptr(st_m),
        _ptr(st_l), _ptr(st_o), _ptr(out), _ptr(lse), _stream(stream)))


PKV_NOALLOC_SCRATCH_BYTES = 64 << 20


def pkv_noalloc_bytes(prob: pkv_problem, max_splits: int) -> int:
    return LIB.pkv_noalloc_bytes(ctypes.byref(prob), max_splits)


def pkv_attend_noalloc(prob: pkv_problem, seq_lens_dev, max_splits: int, q, k_pool, v_pool,
                       block_table, out, lse=None, stream=None) -> None:
    _check("pkv_attend_noalloc", LIB.pkv_attend_noalloc(
        ctypes.byref(prob), _ptr(seq_lens_dev), max_splits, _ptr(q), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(out), _ptr(lse), _stream(stream)))


def pkv_append_kv(prob: pkv_problem, k_new, v_new, block_table, positions_dev, k_pool, v_pool,
                  stream=None) -> None:
    _check("pkv_append_kv", LIB.pkv_append_kv(
        ctypes.byref(prob), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(positions_dev),
        _ptr(k_pool), _ptr(v_pool), _stream(stream)))


def pkv_policy(rules, batch: int, max_len: int):
    """rules: sequence of (b_lo, b_hi, nmax_lo, nmax_hi, path_id, splits)."""
    flat = np.ascontiguousarray(np.asarray(rules, dtype=np.int32).reshape(-1))
    table = pkv_policy_table(len(flat) // 6,
                             flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    path, splits = ctypes.c_int32(), ctypes.c_int32()
    _check("pkv_policy", LIB.pkv_policy(ctypes.byref(table), batch, max_len,
                                        ctypes.byref(path), ctypes.byref(splits)))
    return path.value, splits.value


def pkv_cost_features(prob: pkv_problem, seq_lens_host, path: int, max_splits: int,
                      num_cus: int) -> np.ndarray:
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    scratch = np.empty(max(1, prob.batch), dtype=np.int32)
    out = np.empty(PKV_COST_FEATURES, dtype=np.float32)
    _check("pkv_cost_features", LIB.pkv_cost_features(
        ctypes.byref(prob), lens.ctypes.data, path, max_splits, num_cus, scratch.ctypes.data,
        out.ctypes.data))
    return out


def pkv_policy_model(prob: pkv_problem, candidates, weights, num_cus: int, seq_lens_host):
    """candidates: [(path_id, splits)]; weights: [4][PKV_COST_FEATURES].
    Returns (path_id, splits, predicted_us)."""
    cand = np.ascontiguousarray(np.asarray(candidates, dtype=np.int32).reshape(-1))
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.float32).reshape(-1))
    if w.size != 4 * PKV_COST_FEATURES:
        raise ValueError("weights must be [4][PKV_COST_FEATURES]")
    model = pkv_cost_model(len(cand) // 2, cand.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), num_cus)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    scratch = np.empty(max(1, prob.batch), dtype=np.int32)
    path, splits, pred = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    _check("pkv_policy_model", LIB.pkv_policy_model(
        ctypes.byref(prob), ctypes.byref(model), lens.ctypes.data, scratch.ctypes.data,
        ctypes.byref(path), ctypes.byref(splits), ctypes.byref(pred)))
    return path.value, splits.value, pred.value


def pkv_policy_default(rules, prob: pkv_problem, candidates, weights, num_cus: int,
                       seq_lens_host):
    """rules as for pkv_policy; candidates / weights / num_cus as for
    pkv_policy_model.  Returns (path_id, splits)."""
    flat = np.ascontiguousarray(np.asarray(rules, dtype=np.int32).reshape(-1))
    table = pkv_policy_table(len(flat) // 6,
                             flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    cand = np.ascontiguousarray(np.asarray(candidates, dtype=np.int32).reshape(-1))
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.float32).reshape(-1))
    if w.size != 4 * PKV_COST_FEATURES:
        raise ValueError("weights must be [4][PKV_COST_FEATURES]")
    model = pkv_cost_model(len(cand) // 2, cand.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           w.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), num_cus)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    scratch = np.empty(max(1, prob.batch), dtype=np.int32)
    path, splits = ctypes.c_int32(), ctypes.c_int32()
    _check("pkv_policy_default", LIB.pkv_policy_default(
        ctypes.byref(table), ctypes.byref(model), ctypes.byref(prob), lens.ctypes.data,
        scratch.ctypes.data, ctypes.byref(path), ctypes.byref(splits)))
    return path.value, splits.value


def pkv_balanced_splits(prob: pkv_problem, seq_lens_host, num_cus: int, per_cu: int,
                        max_splits: int) -> int:
    """The CU-balanced workqueue split cap (0 when none fits the budget)."""
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    out = ctypes.c_int32()
    _check("pkv_balanced_splits", LIB.pkv_balanced_splits(
        ctypes.byref(prob), lens.ctypes.data, num_cus, per_cu, max_splits, ctypes.byref(out)))
    return out.value


def decode_plan(plan_host) -> dict:
    """Read a plan buffer (layout in include/pkv.h) into Python lists."""
    w = np.asarray(plan_host.numpy() if hasattr(plan_host, "numpy") else plan_host).view(np.int32)
    assert w[0] == PKV_PLAN_MAGIC
    b = int(w[2])
    h = PKV_PLAN_HEADER_WORDS
    n_tasks, n_buckets = int(w[6]), int(w[7])
    ot, ob, obr = int(w[10]), int(w[11]), int(w[12])
    tasks = w[ot:ot + 4 * n_tasks].reshape(-1, 4)
    psz = int(w[14])
    return {
        "path": PATH_NAMES[int(w[1])],
        "batch": b,
        "splits": int(w[4]),
        "pages_per_split": int(w[5]),
        "n_state_slots": int(w[8]),
        "n_empty_slots": int(w[9]),
        "row_len": w[h:h + b].tolist(),
        "row_pages": w[h + b:h + 2 * b].tolist(),
        "row_nsplit": w[h + 2 * b:h + 3 * b].tolist(),
        "row_task_off": w[h + 3 * b:h + 4 * b + 1].tolist(),
        "tasks": [(int(t[0]), int(t[1]) >> 16, int(t[1]) & 0xFFFF, int(t[2]),
                   -(-int(t[3]) // psz)) for t in tasks],
        "task_token_end": [int(t[3]) for t in tasks],
        "buckets": [tuple(int(x) for x in w[ob + 8 * k:ob + 8 * k + 8]) for k in range(n_buckets)],
        "bucket_rows": w[obr:obr + b].tolist() if n_buckets else [],
        "total_words": int(w[13]),
    }
