"""Cost-model oracle (test infrastructure only): plan features of a
candidate (path, split cap) and the argmin choice of a per-path linear model
of the step time.

A learned cost model is what the PersistentKV summary pages leave as future
work (es page, "Significado y Reivindicaciones" / "Direcciones Futuras";
the paper's own policy, "2. Calibrated adaptive policy", uses
hand-calibrated thresholds).  The features restate counters of
``oracle.planner.plan`` in natural units:

  f0 = 1, f1 = launches per step, f2 = real-KV MB, f3 = merge-state MB,
  f4 = per-CU critical pages: in each split launch the grid items (tasks for
       the workqueue; (row, kv head) for no split; (bucket row, kv head,
       split slot) for the bucket paths, empty slots counting 0 pages) are
       dealt to CUs round-robin in grid order, and the launch contributes the
       largest page total of one CU,
  f5 = grid items / 1000, f6 = non-empty tasks / 1000,
  f7 = pages of the largest task / 100 (the whole longest row for no split).

The model predicts microseconds as w[path] . f; the choice is the argmin.

Parity status: pinned by hand-computed features (tests/test_oracle_cost.py)
and, through them, by the planner pins; ``predict_us`` by hand-computed dot
products and ``choose`` by a hand-worked argmin and a tie (the first
candidate wins).  The fitted weights are measured values and are not pinned.
"""
from __future__ import annotations

from .planner import pages_of, plan

PATH_IDS = {"bucketed": 0, "workqueue": 1, "nosplit": 2, "padded": 3}
N_FEATURES = 8


def launch_grids(seq_lens, num_kv_heads, num_q_heads, head_dim, page_size, splits, path):
    """The plan and, per split launch, the pages of its grid items in order."""
    lens = [int(n) for n in seq_lens]
    p = plan(lens, num_kv_heads, num_q_heads, head_dim, page_size, splits, path)
    if path == "workqueue":
        return p, [[pe - pb for *_, pb, pe in p.tasks]]
    if path == "nosplit":
        return p, [[pages_of(n, page_size) for n in lens for _ in range(num_kv_heads)]]
    pages = {(r, g, s): pe - pb for r, g, s, pb, pe in p.tasks}
    return p, [[pages.get((r, g, s), 0) for r in bk[4] for g in range(num_kv_heads)
                for s in range(splits)] for bk in p.buckets]


def features(seq_lens, num_kv_heads, num_q_heads, head_dim, page_size, splits, path,
             num_cus) -> list:
    if path == "nosplit":
        splits = 1
    p, grids = launch_grids(seq_lens, num_kv_heads, num_q_heads, head_dim, page_size, splits,
                            path)
    crit = 0
    for grid in grids:
        per_cu = [0] * num_cus
        for j, pages in enumerate(grid):
            per_cu[j % num_cus] += pages
        crit += max(per_cu)
    largest = max((pages for grid in grids for pages in grid), default=0)
    return [1.0, float(p.n_launches), p.kv_bytes / 1e6, p.merge_state_bytes / 1e6, float(crit),
            sum(len(g) for g in grids) / 1e3, len(p.tasks) / 1e3, largest / 1e2]


def predict_us(weights, path: str, f) -> float:
    return sum(float(a) * float(x) for a, x in zip(weights[PATH_IDS[path]], f))


def choose(weights, candidates, seq_lens, num_kv_heads, num_q_heads, head_dim, page_size,
           num_cus):
    """Candidate (path, splits) with the smallest predicted time, the first on
    a tie; returns (path, splits, predicted microseconds)."""
    best = None
    for path, s in candidates:
        y = predict_us(weights, path, features(seq_lens, num_kv_heads, num_q_heads, head_dim,
                                               page_size, s, path, num_cus))
        if best is None or y < best[2]:
            best = (path, s, y)
    return best
