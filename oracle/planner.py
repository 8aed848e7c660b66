"""Integer oracle for the decode planner (test infrastructure only).

Parity status: pinned by closed forms and invariants in
``tests/test_oracle_planner.py`` (partition of every row's pages, task counts,
launches per step = 2 x distinct lengths for exact buckets vs 2 for the compact
workqueue, which reproduces the 16.00 -> 2.00 launches/step of the pages'
"Results" section at B=8 with distinct lengths).

What it restates (PersistentKV summary pages, "Methodology / 1. Native
block-table decode engine"):

* Row-local bounds: tile counts and split ranges come from each row's real
  length N_i; a tile is one KV page, so row i has T_i = ceil(N_i / P) pages.
* Sequence splitting: a row's pages are cut into disjoint contiguous ranges.
* Compact workqueue: one 1-D list holding only the non-empty
  (row, kv-head, split) intervals.
* Exact-length buckets (the alternative the pages compare against): rows with
  the same length form a bucket launched as one rectangular grid; slots past a
  bucket's split count are empty and write neutral state.

Readings where the pages are silent (each listed in the design notes):
* workqueue split granule is shared by the batch: pps = max(1, ceil(T_max / S)),
  row i gets ceil(T_i / pps) splits;
* a bucket's granule is pps_b = max(1, ceil(T_b / S)), ceil(T_b / pps_b) splits;
* tasks are ordered (row, kv_head, split); buckets by ascending length, rows
  ascending inside a bucket;
* the no-split path has one task per (row, kv_head) of every non-empty row;
* padded power-of-two buckets (the coarse-padding alternative the pages'
  "Problem statement" contrasts with): rows are grouped by their page count
  rounded up to a power of two, the bucket's granule is
  pps_b = max(1, ceil(T_pad / S)) pages of the padded length, and row i keeps
  its row-local bound -- ceil(T_i / pps_b) non-empty splits; the bucket's
  other slots are empty (neutral state).  Empty rows form their own bucket.
"""
from __future__ import annotations

from dataclasses import dataclass, field


def pages_of(n: int, page_size: int) -> int:
    return -(-int(n) // page_size)


@dataclass
class Plan:
    path: str
    tasks: list = field(default_factory=list)  # (row, kv_head, split, page_begin, page_end)
    row_pages: list = field(default_factory=list)
    row_nsplit: list = field(default_factory=list)
    row_task_off: list = field(default_factory=list)
    buckets: list = field(default_factory=list)  # (length, pages, pps, nsplit, rows tuple)
    pages_per_split: int = 0
    n_launches: int = 0
    n_state_slots: int = 0
    n_empty_slots: int = 0
    kv_bytes: int = 0
    merge_state_bytes: int = 0


def plan(seq_lens, num_kv_heads: int, num_q_heads: int, head_dim: int, page_size: int,
         splits: int, path: str, elem_bytes: int = 2) -> Plan:
    """Plan one decode step.  ``path`` is "workqueue", "bucketed", "padded" or "nosplit"."""
    lens = [int(n) for n in seq_lens]
    b = len(lens)
    hkv = num_kv_heads
    grp = num_q_heads // num_kv_heads
    pages = [pages_of(n, page_size) for n in lens]
    p = Plan(path=path, row_pages=pages)
    p.kv_bytes = sum(lens) * hkv * head_dim * 2 * elem_bytes

    if path == "workqueue":
        t_max = max(pages) if pages else 0
        pps = max(1, -(-t_max // splits))
        p.pages_per_split = pps
        nsplit = [-(-t // pps) for t in pages]
        p.row_nsplit = nsplit
        off = 0
        for i in range(b):
            p.row_task_off.append(off)
            for g in range(hkv):
                for s in range(nsplit[i]):
                    p.tasks.append((i, g, s, s * pps, min((s + 1) * pps, pages[i])))
            off += hkv * nsplit[i]
        p.row_task_off.append(off)
        p.n_state_slots = len(p.tasks)
        p.n_empty_slots = 0
        p.n_launches = 1 + (1 if p.tasks else 0)
    elif path == "bucketed":
        by_len = {}
        for i, n in enumerate(lens):
            by_len.setdefault(n, []).append(i)
        nsplit_row = [0] * b
        for n in sorted(by_len):
            t_b = pages_of(n, page_size)
            pps = max(1, -(-t_b // splits))
            ns = -(-t_b // pps)
            rows = tuple(sorted(by_len[n]))
            p.buckets.append((n, t_b, pps, ns, rows))
            for i in rows:
                nsplit_row[i] = ns
                for g in range(hkv):
                    for s in range(ns):
                        p.tasks.append((i, g, s, s * pps, min((s + 1) * pps, t_b)))
            p.n_state_slots += len(rows) * hkv * splits
            p.n_empty_slots += len(rows) * hkv * (splits - ns)
        p.row_nsplit = nsplit_row
        p.n_launches = 2 * len(p.buckets)
    elif path == "padded":
        by_pad = {}
        for i, t in enumerate(pages):
            pad = 0 if t == 0 else 1 << (t - 1).bit_length()
            by_pad.setdefault(pad, []).append(i)
        nsplit_row = [0] * b
        for pad in sorted(by_pad):
            pps = max(1, -(-pad // splits))
            rows = tuple(sorted(by_pad[pad]))
            p.buckets.append((-1, pad, pps, -(-pad // pps), rows))
            for i in rows:
                ns = -(-pages[i] // pps)
                nsplit_row[i] = ns
                for g in range(hkv):
                    for s in range(ns):
                        p.tasks.append((i, g, s, s * pps, min((s + 1) * pps, pages[i])))
                p.n_empty_slots += hkv * (splits - ns)
            p.n_state_slots += len(rows) * hkv * splits
        p.row_nsplit = nsplit_row
        p.n_launches = 2 * len(p.buckets)
    elif path == "nosplit":
        for i in range(b):
            if pages[i]:
                for g in range(hkv):
                    p.tasks.append((i, g, 0, 0, pages[i]))
        p.row_nsplit = [1 if t else 0 for t in pages]
        p.n_launches = 1
    else:
        raise ValueError(path)
    p.merge_state_bytes = 2 * p.n_state_slots * grp * (head_dim + 2) * 4
    return p
