"""Policy-table oracle (test infrastructure only).

The PersistentKV summary pages ("2. Calibrated adaptive policy") describe a
hand-calibrated rule keyed on batch size B and the longest context N_max that
picks the execution path.  Restated here as an ordered table whose first
matching rule wins: a rule (b_lo, b_hi, n_lo, n_hi, path, splits) matches when
b_lo <= B <= b_hi and n_lo <= N_max <= n_hi.  No matching rule -> None.

Parity status: pinned structurally (first match, inclusive bounds, no match)
in ``tests/test_oracle_planner.py``; the pages' RTX 3060 thresholds do not carry
over to other hardware, so no threshold value is pinned.
"""
from __future__ import annotations


def choose(rules, batch: int, max_len: int):
    for b_lo, b_hi, n_lo, n_hi, path, splits in rules:
        if b_lo <= batch <= b_hi and n_lo <= max_len <= n_hi:
            return path, splits
    return None
