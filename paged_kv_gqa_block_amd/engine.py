"""One decode step through libpkv: buffers from torch, work in the library.

``DecodeStep`` owns the per-step buffers (pinned host plan, device plan,
partial states, output) for one problem shape and one path, and calls the C
ABI in the documented order: pkv_plan -> pkv_decode -> pkv_merge.  torch only
allocates memory and supplies the stream.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from . import _lib
from ._lib import (PATH_IDS, PATH_NAMES, PKV_NOSPLIT, PKV_WORKQUEUE, make_problem, pkv_decode,
                   pkv_decode_device, pkv_merge, pkv_merge_device, pkv_plan, pkv_plan_bytes,
                   pkv_plan_device, pkv_policy)

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}
POLICY_TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "policy_table.json")
COST_MODEL_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_model.json")


def problem_from_workload(w: dict, kernel: str = "auto") -> _lib.pkv_problem:
    spec = w["spec"]
    return make_problem(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                        spec.page_size, int(w["k_pool"].shape[0]),
                        int(w["block_table"].shape[1]), spec.dtype, w["scale"], kernel)


def to_device(w: dict, device="cuda") -> dict:
    """Copy a generated workload's tensors to the GPU (inputs resident in HBM)."""
    out = dict(w)
    for key in ("q", "k_pool", "v_pool", "block_table", "seq_lens"):
        out[key] = w[key].to(device).contiguous()
    out["seq_lens_host"] = w["seq_lens"].numpy().astype(np.int32).copy()
    return out


class DecodeStep:
    """Buffers and calls for one (problem, path, split cap)."""

    def __init__(self, prob: _lib.pkv_problem, path, splits: int, device="cuda"):
        self.prob = prob
        self.path = PATH_IDS[path] if isinstance(path, str) else path
        self.splits = int(splits)
        self.device = torch.device(device)
        nbytes = pkv_plan_bytes(prob, self.path, self.splits)
        if nbytes == 0:
            raise _lib.PkvError("pkv_plan_bytes", _lib.PKV_EINVAL, "invalid problem")
        pin = self.device.type == "cuda"
        self.plan_host = torch.zeros(nbytes // 4, dtype=torch.int32, pin_memory=pin)
        self.plan_dev = torch.zeros(nbytes // 4, dtype=torch.int32, device=self.device)
        self.info = None
        g = prob.num_q_heads // prob.num_kv_heads
        d = prob.head_dim
        dt = torch.bfloat16 if prob.dtype == _lib.PKV_BF16 else torch.float16
        self.out = torch.empty(prob.batch, prob.num_q_heads, d, dtype=dt, device=self.device)
        self.lse = torch.empty(prob.batch, prob.num_q_heads, dtype=torch.float32,
                               device=self.device)
        # Upper bound of state slots: every row at the split cap.
        slots = prob.batch * prob.num_kv_heads * (1 if self.path == PKV_NOSPLIT else self.splits)
        self.st_m = torch.empty(max(slots, 1), g, dtype=torch.float32, device=self.device)
        self.st_l = torch.empty(max(slots, 1), g, dtype=torch.float32, device=self.device)
        self.st_o = torch.empty(max(slots, 1), g, d, dtype=torch.float32, device=self.device)

    def plan(self, seq_lens_host: np.ndarray, stream=None) -> _lib.pkv_plan_info:
        self.info = pkv_plan(self.prob, np.ascontiguousarray(seq_lens_host, dtype=np.int32),
                             self.path, self.splits, self.plan_host, self.plan_dev, stream=stream)
        return self.info

    def decode(self, w: dict, stream=None) -> None:
        pkv_decode(self.prob, self.plan_host, self.plan_dev, w["q"], w["k_pool"], w["v_pool"],
                   w["block_table"], w["seq_lens"], self.st_m, self.st_l, self.st_o, self.out,
                   self.lse, stream=stream)

    def merge(self, stream=None) -> None:
        pkv_merge(self.prob, self.plan_host, self.plan_dev, self.st_m, self.st_l, self.st_o,
                  self.out, self.lse, stream=stream)

    def run(self, w: dict, stream=None):
        self.decode(w, stream)
        self.merge(stream)
        return self.out, self.lse

    def bind(self, w: dict, stream=None) -> tuple:
        """pkv_decode and pkv_merge of this step on workload buffers `w`, with
        their arguments marshalled once (see ``run_bound``)."""
        st = stream if stream is not None else torch.cuda.current_stream()
        dec = _lib.bind_call("pkv_decode", self.prob, self.plan_host, self.plan_dev, w["q"],
                             w["k_pool"], w["v_pool"], w["block_table"], w["seq_lens"],
                             self.st_m, self.st_l, self.st_o, self.out, self.lse, st)
        mrg = _lib.bind_call("pkv_merge", self.prob, self.plan_host, self.plan_dev, self.st_m,
                             self.st_l, self.st_o, self.out, self.lse, st)
        return dec, mrg

    def run_bound(self, bound: tuple) -> None:
        """The same two calls as ``run`` with pre-marshalled arguments: the
        host enqueues a step in a few microseconds, so timing loops of short
        steps measure the device, not the Python binding."""
        _lib.call_bound(bound[0])
        _lib.call_bound(bound[1])

    def decode_bound(self, bound: tuple) -> None:
        _lib.call_bound(bound[0])


class _PersistentStepBuffers:
    """Output and partial-state buffers of a persistent-grid workqueue step
    (room for B * Hkv * S states: the most any length mix can need)."""

    def __init__(self, prob: _lib.pkv_problem, splits: int, device="cuda"):
        self.prob = prob
        self.splits = int(splits)
        self.device = torch.device(device)
        g = prob.num_q_heads // prob.num_kv_heads
        d = prob.head_dim
        dt = torch.bfloat16 if prob.dtype == _lib.PKV_BF16 else torch.float16
        slots = prob.batch * prob.num_kv_heads * self.splits
        self.out = torch.empty(prob.batch, prob.num_q_heads, d, dtype=dt, device=self.device)
        self.lse = torch.empty(prob.batch, prob.num_q_heads, dtype=torch.float32,
                               device=self.device)
        self.st_m = torch.empty(slots, g, dtype=torch.float32, device=self.device)
        self.st_l = torch.empty(slots, g, dtype=torch.float32, device=self.device)
        self.st_o = torch.empty(slots, g, d, dtype=torch.float32, device=self.device)


class DeviceStep(_PersistentStepBuffers):
    """Device-planned workqueue step: plan, split and merge all on the GPU.

    ``run`` enqueues pkv_plan_device -> pkv_decode_device -> pkv_merge_device on
    one stream with no host work, so the three launches can be captured once in
    a HIP graph and replayed while the device lengths change.
    """

    def __init__(self, prob: _lib.pkv_problem, splits: int, device="cuda"):
        super().__init__(prob, splits, device)
        nbytes = pkv_plan_bytes(prob, PKV_WORKQUEUE, self.splits)
        if nbytes == 0:
            raise _lib.PkvError("pkv_plan_bytes", _lib.PKV_EINVAL, "invalid problem")
        self.plan_dev = torch.zeros(nbytes // 4, dtype=torch.int32, device=self.device)
        self.bad_rows = torch.zeros(1, dtype=torch.int32, device=self.device)

    def run(self, w: dict, stream=None):
        pkv_plan_device(self.prob, w["seq_lens"], self.splits, self.plan_dev,
                        bad_rows_dev=self.bad_rows, stream=stream)
        pkv_decode_device(self.prob, self.plan_dev, self.splits, w["q"], w["k_pool"],
                          w["v_pool"], w["block_table"], self.st_m, self.st_l, self.st_o,
                          stream=stream)
        pkv_merge_device(self.prob, self.plan_dev, self.st_m, self.st_l, self.st_o, self.out,
                         self.lse, stream=stream)
        return self.out, self.lse


class SelfPlannedStep(_PersistentStepBuffers):
    """Self-planned workqueue step: the device-planned step in two launches.

    ``run`` enqueues pkv_decode_selfplan -> pkv_merge_selfplan: the split and
    merge kernels derive the workqueue of the device lengths themselves, so
    there is no planner launch and no plan buffer, only a one-word claim
    counter (zeroed here once; the merge leaves it zeroed).
    """

    def __init__(self, prob: _lib.pkv_problem, splits: int, device="cuda"):
        super().__init__(prob, splits, device)
        self.counter = torch.zeros(1, dtype=torch.int32, device=self.device)

    def run(self, w: dict, stream=None):
        _lib.pkv_decode_selfplan(self.prob, w["seq_lens"], self.splits, self.counter, w["q"],
                                 w["k_pool"], w["v_pool"], w["block_table"], self.st_m,
                                 self.st_l, self.st_o, stream=stream)
        _lib.pkv_merge_selfplan(self.prob, w["seq_lens"], self.splits, self.counter, self.st_m,
                                self.st_l, self.st_o, self.out, self.lse, stream=stream)
        return self.out, self.lse


def load_policy_table(path: str = POLICY_TABLE_PATH):
    """Rules [(b_lo, b_hi, nmax_lo, nmax_hi, path_id, splits)] from the JSON table."""
    with open(path) as f:
        doc = json.load(f)
    return [(r["b_lo"], r["b_hi"], r["nmax_lo"], r["nmax_hi"], PATH_IDS[r["path"]], r["splits"])
            for r in doc["rules"]]


def choose(rules, batch: int, max_len: int):
    """Path name and split cap from the calibrated table (C-ABI pkv_policy)."""
    path, splits = pkv_policy(rules, batch, max_len)
    return PATH_NAMES[path], splits


def split_kernel_of(prob: _lib.pkv_problem) -> str:
    """The split-kernel variant pkv_decode runs for this problem: the explicit
    choice, else the library's AUTO rule (matrix cores for d = 128, vector ALU
    for 64).  The matrix-core kernel for G > 8 is a variant of its own (two
    resident workgroups per CU instead of three, deeper prefetch), with its
    own cost model."""
    if prob.kernel == _lib.PKV_KERNEL_VALU or (prob.kernel == _lib.PKV_KERNEL_AUTO
                                               and prob.head_dim != 128):
        return "valu"
    return "mfma" if prob.num_q_heads // prob.num_kv_heads <= 8 else "mfma_g16"


def load_cost_model(path: str = COST_MODEL_PATH):
    """(candidates [(path_id, splits)], {split kernel: weights [4][PKV_COST_FEATURES]},
    num_cus).  The model has one weight matrix per split kernel."""
    with open(path) as f:
        doc = json.load(f)
    cands = [(PATH_IDS[c["path"]], c["splits"]) for c in doc["candidates"]]
    weights = {}
    for kernel, rows in doc["weights"].items():
        w = np.zeros((4, _lib.PKV_COST_FEATURES), dtype=np.float32)
        for name, row in rows.items():
            w[PATH_IDS[name]] = np.asarray(row, dtype=np.float32)
        weights[kernel] = w
    return cands, weights, int(doc["num_cus"])


def choose_model(model, prob: _lib.pkv_problem, seq_lens_host):
    """Path name, split cap and predicted µs from the learned cost model
    (C-ABI pkv_policy_model, with the weights of the problem's split kernel)."""
    cands, weights, num_cus = model
    path, splits, pred = _lib.pkv_policy_model(prob, cands, weights[split_kernel_of(prob)],
                                               num_cus, seq_lens_host)
    return PATH_NAMES[path], splits, pred


# Candidates of the default policy's cost-model leg (B >= 2): the compact
# workqueue at each split cap, and the single-pass kernel.  On the calibration
# and held-out draws of every sweep and trace workload the full candidate list
# picks the same (path, split cap) at B >= 2, at a third of the host time.
DEFAULT_MODEL_PATHS = (PKV_WORKQUEUE, PKV_NOSPLIT)


def choose_default(rules, model, prob: _lib.pkv_problem, seq_lens_host):
    """Path name and split cap of the engine's default policy
    (pkv_policy_default): the calibrated table for one row, the learned cost
    model (workqueue and no-split candidates, and the CU-balanced workqueue
    caps the library adds) for several."""
    cands, weights, num_cus = model
    cands = [c for c in cands if c[0] in DEFAULT_MODEL_PATHS]
    path, splits = _lib.pkv_policy_default(rules, prob, cands, weights[split_kernel_of(prob)],
                                           num_cus, seq_lens_host)
    return PATH_NAMES[path], splits


def validate_inputs(w: dict) -> None:
    """Host-side checks that the tensors match what the kernels assume.

    Shapes, dtypes and contiguity of q / pools / block table / lengths, every
    length within the table's capacity, and every block-table entry that a
    row uses inside [0, num_pool_pages).  Raises ValueError.
    """
    spec = w["spec"]
    q, kp, vp, bt, sl = w["q"], w["k_pool"], w["v_pool"], w["block_table"], w["seq_lens"]
    dt = TORCH_DTYPE[spec.dtype]
    b, hq, hkv, d, p = (spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                        spec.page_size)
    if tuple(q.shape) != (b, hq, d) or q.dtype != dt:
        raise ValueError(f"q: {tuple(q.shape)} {q.dtype}")
    for name, t in (("k_pool", kp), ("v_pool", vp)):
        if t.dim() != 4 or tuple(t.shape[1:]) != (hkv, p, d) or t.dtype != dt:
            raise ValueError(f"{name}: {tuple(t.shape)} {t.dtype}")
    if kp.shape[0] != vp.shape[0]:
        raise ValueError("K and V pools differ in page count")
    if bt.dim() != 2 or bt.shape[0] != b or bt.dtype != torch.int32:
        raise ValueError(f"block_table: {tuple(bt.shape)} {bt.dtype}")
    if tuple(sl.shape) != (b,) or sl.dtype != torch.int32:
        raise ValueError(f"seq_lens: {tuple(sl.shape)} {sl.dtype}")
    for t in (q, kp, vp, bt, sl):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    lens = sl.cpu().numpy()
    btn = bt.cpu().numpy()
    cap = btn.shape[1] * p
    pool = kp.shape[0]
    for i, n in enumerate(lens):
        if n < 0 or n > cap:
            raise ValueError(f"row {i}: length {n} outside [0, {cap}]")
        used = btn[i, :(int(n) + p - 1) // p]
        if used.size and (used.min() < 0 or used.max() >= pool):
            raise ValueError(f"row {i}: block-table entry outside [0, {pool})")
