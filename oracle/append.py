"""KV append oracle (test infrastructure only).

Before attention, a decode step stores the new token's key and value of every
row in the paged pool: token position p of row i lives in pool page
``block_table[i][p // P]`` at slot ``p % P`` -- the same addressing the
attention reads (PersistentKV summary pages, "Methodology / 1. Native
block-table decode engine", *Layout*: pages are used in place through the
block table).  The pages do not describe the append; this is its plain
definition.  Rows with a negative position are inactive and write nothing.

Parity status: pinned by tests/test_oracle.py (writes land at the addressed
slot; nothing else changes; append of N tokens one by one equals the pool the
workload generator builds).
"""
from __future__ import annotations

import numpy as np


def append_kv(k_pool, v_pool, block_table, positions, k_new, v_new, page_size: int):
    """Return copies of the pools with row i's new K/V written at positions[i]."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for i, p in enumerate(np.asarray(positions)):
        p = int(p)
        if p < 0:
            continue
        page = int(block_table[i][p // page_size])
        k[page, :, p % page_size, :] = k_new[i]
        v[page, :, p % page_size, :] = v_new[i]
    return k, v
