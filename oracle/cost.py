"""Cost-model oracle (test infrastructure only): plan features of a
candidate (path, split cap) and the argmin choice of a per-path linear model
of log2 step time.

A learned cost model is what the PersistentKV summary pages leave as future
work (section "Conclusion"; the paper's own policy, "2. Calibrated adaptive
policy", uses hand-calibrated thresholds).  The features restate the plan
counters of ``oracle.planner.plan`` -- tasks, launches, state slots, merge
state bytes, real-KV bytes and the longest task -- in fp64:

  f0 = 1, f1 = log2 B, f2 = log2 max(1, N_max), f3 = log2 max(1, mean N),
  f4 = log2 S (0 for the no-split path), f5 = log2 max(1, tasks),
  f6 = launches, f7 = log2 max(1, grid items), f8 = log2(1 + state bytes),
  f9 = log2 max(1, KV bytes), f10 = log2 max(1, longest task in pages),

grid items being the task count (workqueue), B * Hkv (no split) or the state
slots (bucket paths).  The model predicts log2 microseconds as w[path] . f.

Parity status: pinned by hand-computed features (tests/test_oracle_cost.py)
and, through them, by the planner pins; the fitted weights are measured
values and are not pinned.
"""
from __future__ import annotations

import math

from .planner import plan

PATH_IDS = {"bucketed": 0, "workqueue": 1, "nosplit": 2, "padded": 3}
N_FEATURES = 11


def _lg(x: float) -> float:
    return math.log2(max(1.0, float(x)))


def features(seq_lens, num_kv_heads: int, num_q_heads: int, head_dim: int, page_size: int,
             splits: int, path: str) -> list:
    lens = [int(n) for n in seq_lens]
    b = len(lens)
    p = plan(lens, num_kv_heads, num_q_heads, head_dim, page_size, splits, path)
    n_tasks = len(p.tasks)
    if path == "workqueue":
        items = n_tasks
    elif path == "nosplit":
        items = b * num_kv_heads
    else:
        items = p.n_state_slots
    longest = max((pe - pb for *_, pb, pe in p.tasks), default=0)
    return [1.0, _lg(b), _lg(max(lens)), _lg(sum(lens) / b),
            _lg(1 if path == "nosplit" else splits), _lg(n_tasks), float(p.n_launches),
            _lg(items), math.log2(1.0 + p.merge_state_bytes), _lg(p.kv_bytes), _lg(longest)]


def predict_log2_us(weights, path: str, f) -> float:
    w = weights[PATH_IDS[path]]
    return sum(float(a) * float(x) for a, x in zip(w, f))


def choose(weights, candidates, seq_lens, num_kv_heads, num_q_heads, head_dim, page_size):
    """Candidate (path, splits) with the smallest predicted time, the first on
    a tie; returns (path, splits, predicted log2 microseconds)."""
    best = None
    for path, s in candidates:
        y = predict_log2_us(weights, path, features(seq_lens, num_kv_heads, num_q_heads,
                                                     head_dim, page_size, s, path))
        if best is None or y < best[2]:
            best = (path, s, y)
    return best
