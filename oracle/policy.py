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

Parity status: pinned structurally (first match, inclusive bounds, no match)
in ``tests/test_oracle_planner.py``; the pages' RTX 3060 thresholds do not carry
over to other hardware, so no threshold value is pinned.  ``choose_default``
is pinned by a hand-worked case on each side of its B = 1 / B >= 2 split
(tests/test_oracle_cost.py).
"""
from __future__ import annotations


def choose(rules, batch: int, max_len: int):
    for b_lo, b_hi, n_lo, n_hi, path, splits in rules:
        if b_lo <= batch <= b_hi and n_lo <= max_len <= n_hi:
            return path, splits
    return None


def choose_default(rules, weights, candidates, seq_lens, num_kv_heads, num_q_heads, head_dim,
                   page_size, num_cus):
    """(path, splits): the table for one row, the cost model for several."""
    from . import cost

    lens = [int(n) for n in seq_lens]
    if len(lens) == 1:
        return choose(rules, 1, lens[0])
    path, splits, _ = cost.choose(weights, candidates, lens, num_kv_heads, num_q_heads,
                                  head_dim, page_size, num_cus)
    return path, splits
