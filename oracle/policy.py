"""Policy-table oracle (test infrastructure only).

The PersistentKV summary pages ("2. Calibrated adaptive policy") describe a
hand-calibrated rule keyed on batch size B and the longest context N_max that
picks the execution path.  Restated here as an ordered table whose first
matching rule wins: a rule (b_lo, b_hi, n_lo, n_hi, path, splits) matches when
b_lo <= B <= b_hi and n_lo <= N_max <= n_hi.  No matching rule -> None.

``choose_default`` is the engine's default choice: the table's rule for
(1, N_1) when there is one row (its length fixes the workload), else the
learned cost model's argmin (``oracle.cost.choose``), which sees the length
mix that the table's key does not ("Significado y Reivindicaciones" /
"Direcciones Futuras", es page: a learned cost model for the thresholds).
The model scores its listed candidates and then the CU-balanced workqueue
split caps (``balanced_splits``: the largest cap whose compact workqueue
holds at most 1, resp. 2, tasks per compute unit), which the engine adds
because the split count is the policy's choice and an even share of tasks
per CU is what the per-CU feature rewards.

Parity status: pinned structurally (first match, inclusive bounds, no match)
in ``tests/test_oracle_planner.py``; the pages' RTX 3060 thresholds do not carry
over to other hardware, so no threshold value is pinned.  ``choose_default``
is pinned by a hand-worked case on each side of its B = 1 / B >= 2 split and
one where a balanced cap wins; ``balanced_splits`` by hand-counted task lists
(tests/test_oracle_cost.py).
"""
from __future__ import annotations


def choose(rules, batch: int, max_len: int):
    for b_lo, b_hi, n_lo, n_hi, path, splits in rules:
        if b_lo <= batch <= b_hi and n_lo <= max_len <= n_hi:
            return path, splits
    return None


BALANCED_TASKS_PER_CU = (1, 2)


def balanced_splits(seq_lens, num_kv_heads, num_q_heads, head_dim, page_size, num_cus, per_cu,
                    max_splits):
    """Largest split cap S in 1..max_splits whose workqueue plan has at most
    per_cu * num_cus tasks; 0 if there is none.  Counts the tasks of every
    cap's plan (``oracle.planner.plan``)."""
    from .planner import plan

    lens = [int(n) for n in seq_lens]
    best = 0
    for s in range(1, max_splits + 1):
        p = plan(lens, num_kv_heads, num_q_heads, head_dim, page_size, s, "workqueue")
        if len(p.tasks) <= per_cu * num_cus:
            best = s
    return best


def choose_default(rules, weights, candidates, seq_lens, num_kv_heads, num_q_heads, head_dim,
                   page_size, num_cus):
    """(path, splits): the table for one row; for several, the cost model's
    argmin over the candidates followed by the balanced workqueue caps not
    already among them (the earlier of equal predictions wins)."""
    from . import cost

    lens = [int(n) for n in seq_lens]
    if len(lens) == 1:
        return choose(rules, 1, lens[0])
    listed = [(p, int(s)) for p, s in candidates]
    caps = [s for p, s in listed if p == "workqueue"]
    extra = []
    for per_cu in BALANCED_TASKS_PER_CU:
        s = balanced_splits(lens, num_kv_heads, num_q_heads, head_dim, page_size, num_cus,
                            per_cu, max(caps)) if caps else 0
        if s > 0 and ("workqueue", s) not in listed + extra:
            extra.append(("workqueue", s))
    path, splits, _ = cost.choose(weights, listed + extra, lens, num_kv_heads, num_q_heads,
                                  head_dim, page_size, num_cus)
    return path, splits
