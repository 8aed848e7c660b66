"""fp64 gather-then-softmax oracle (test infrastructure only; see package docstring).

Parity status: pinned.  ``tests/test_oracle.py`` checks ``attention`` against
torch's dense scaled-dot-product attention on contiguous K/V that were then
scattered into a shuffled page pool, against closed forms (one token, constant
keys, zero query, a hand-worked two-token example in ``tests/golden/``), and
against invariants (page permutation, score shift, linearity in V); it
checks ``split_state`` + ``merge`` against the unsplit result for random
partitions; and it checks ``split_states_for_plan`` by merging the states of
every task of ``oracle.plan`` (all four paths, lengths off page boundaries,
rows shorter than the split cap, empty rows, NaN page tails) back into the
unsplit result.
"""
from __future__ import annotations

import numpy as np


def decode_values(arr, dtype: str) -> np.ndarray:
    """Stored fp16 / bf16 values -> float64.

    fp16 arrives as ``numpy.float16``; bf16 arrives as raw uint16 bit patterns.
    A bf16 value is the upper 16 bits of the float32 with the same bits.
    """
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather_row(k_pool, v_pool, block_table_row, n: int, kv_head: int, page_size: int,
               dtype: str, t0: int = 0, t1: int | None = None):
    """K and V of tokens [t0, t1) of one row and one KV head, in token order.

    Token t lives in pool page ``block_table_row[t // P]`` at slot ``t % P``;
    nothing is repacked, each token is looked up through the table.
    """
    if t1 is None:
        t1 = n
    t = np.arange(t0, t1)
    pages = np.asarray(block_table_row)[t // page_size]
    slots = t % page_size
    k = decode_values(k_pool[pages, kv_head, slots, :], dtype)
    v = decode_values(v_pool[pages, kv_head, slots, :], dtype)
    return k, v


def attention(q, k_pool, v_pool, block_table, seq_lens, scale: float, page_size: int,
              dtype: str, rows=None):
    """Decode attention output and natural-log LSE for every (row, q-head).

    For row i and query head h, the KV head is g = h // G (contiguous groups of
    G = Hq / Hkv query heads).  Over the row's real tokens t < N_i:
    x_t = scale * <q_h, k_t>, out = sum_t softmax(x)_t v_t, lse = log sum exp x.
    A row with N_i = 0 gives out = 0 and lse = -inf.
    Returns (out [B][Hq][d], lse [B][Hq]) in float64; ``rows`` limits the work
    to a subset of rows (others stay 0 / -inf).
    """
    qd = decode_values(q, dtype)
    b, hq, d = qd.shape
    hkv = k_pool.shape[1]
    assert hq % hkv == 0
    grp = hq // hkv
    out = np.zeros((b, hq, d), dtype=np.float64)
    lse = np.full((b, hq), -np.inf, dtype=np.float64)
    for i in (range(b) if rows is None else rows):
        n = int(seq_lens[i])
        if n == 0:
            continue
        for g in range(hkv):
            k, v = gather_row(k_pool, v_pool, block_table[i], n, g, page_size, dtype)
            for h in range(g * grp, (g + 1) * grp):
                x = scale * (k @ qd[i, h])
                m = x.max()
                e = np.exp(x - m)
                s = e.sum()
                out[i, h] = (e @ v) / s
                lse[i, h] = m + np.log(s)
    return out, lse


def split_state(q, k_pool, v_pool, block_table_row, q_row: int, kv_head: int, t0: int, t1: int,
                scale: float, page_size: int, dtype: str, group: int):
    """Partial online-softmax state of tokens [t0, t1) for the G heads of one KV head.

    Returns (m [G], l [G], o [G][d]) with m = max score, l = sum exp(x - m) and
    o = sum exp(x - m) v (unnormalised).  An empty range is the neutral state
    (-inf, 0, 0), which the merge ignores.
    """
    qd = decode_values(q[q_row, kv_head * group:(kv_head + 1) * group], dtype)
    d = qd.shape[-1]
    if t1 <= t0:
        return (np.full(group, -np.inf), np.zeros(group), np.zeros((group, d)))
    k, v = gather_row(k_pool, v_pool, block_table_row, t1, kv_head, page_size, dtype, t0, t1)
    x = scale * (qd @ k.T)  # [G][n]
    m = x.max(axis=1)
    e = np.exp(x - m[:, None])
    return m, e.sum(axis=1), e @ v


def merge(ms, ls, os):
    """Exact combination of partial states along the first axis.

    ms, ls: [S, ...]; os: [S, ..., d].  M = max_s m_s, w_s = exp(m_s - M)
    (w_s = 0 for a neutral state), L = sum_s w_s l_s, out = sum_s w_s o_s / L,
    lse = M + log L.  If every state is neutral: out = 0, lse = -inf.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    os = np.asarray(os, dtype=np.float64)
    big_m = ms.max(axis=0)
    finite = np.isfinite(big_m)
    safe_m = np.where(finite, big_m, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - safe_m), 0.0)
    big_l = (w * ls).sum(axis=0)
    num = (w[..., None] * os).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(finite[..., None], num / np.where(finite, big_l, 1.0)[..., None], 0.0)
        lse = np.where(finite, safe_m + np.log(np.where(finite, big_l, 1.0)), -np.inf)
    return out, lse


def split_states_for_plan(q, k_pool, v_pool, block_table, tasks, scale: float, page_size: int,
                          dtype: str, group: int, seq_lens):
    """States for a list of (row, kv_head, split, page_begin, page_end) tasks.

    Token range of a task: [page_begin * P, min(page_end * P, N_row)).
    Returns m [n][G], l [n][G], o [n][G][d].
    """
    d = q.shape[-1]
    n = len(tasks)
    m = np.empty((n, group))
    l = np.empty((n, group))
    o = np.empty((n, group, d))
    for j, (row, g, _s, pb, pe) in enumerate(tasks):
        t0 = pb * page_size
        t1 = min(pe * page_size, int(seq_lens[row]))
        m[j], l[j], o[j] = split_state(q, k_pool, v_pool, block_table[row], row, g, t0, t1,
                                       scale, page_size, dtype, group)
    return m, l, o


def round_to_f16(x) -> np.ndarray:
    """float64 -> nearest-even fp16 value, returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest-even bf16 value, returned as float64.

    Rounds to float32 first (nearest-even), then keeps the top 16 bits with
    round-half-to-even on the dropped 16 bits.  NaN is not expected here.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (rounded << np.uint64(16)).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)
