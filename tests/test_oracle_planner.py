"""Pins for the planner and policy oracles (CPU only): closed forms and invariants."""
import json
import os

import numpy as np
import pytest

from oracle.planner import pages_of, plan
from oracle.policy import choose

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_partition(p, lens, hkv, page_size):
    """Every (row, kv_head) has tasks that tile [0, T_i) exactly, none empty."""
    by_key = {}
    for row, g, s, pb, pe in p.tasks:
        assert pe > pb, "empty task"
        by_key.setdefault((row, g), []).append((s, pb, pe))
    for i, n in enumerate(lens):
        t = pages_of(n, page_size)
        for g in range(hkv):
            items = by_key.get((i, g), [])
            if t == 0:
                assert not items
                continue
            items.sort()
            assert [s for s, _, _ in items] == list(range(len(items)))
            assert items[0][1] == 0 and items[-1][2] == t
            for (_, _, e0), (_, b1, _) in zip(items[:-1], items[1:]):
                assert e0 == b1


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("path", ["workqueue", "bucketed", "nosplit", "padded"])
def test_plan_partitions_rows(seed, path):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 9))
    lens = rng.integers(0, 700, size=b)
    lens[rng.random(b) < 0.2] = 0
    hkv = int(rng.choice([1, 2, 8]))
    s = int(rng.choice([1, 3, 4, 32]))
    p = plan(lens, hkv, hkv * 4, 64, 16, s, path)
    _check_partition(p, lens, hkv, 16)
    pages = [pages_of(n, 16) for n in lens]
    assert p.row_pages == pages
    if path != "nosplit":
        assert all(ns <= s for ns in p.row_nsplit)
    assert len(p.tasks) == hkv * sum(p.row_nsplit)
    assert p.kv_bytes == int(sum(int(n) for n in lens)) * hkv * 64 * 2 * 2


def test_workqueue_closed_forms():
    lens = [2048 * 16, 100 * 16, 1, 0, 31 * 16 + 5]
    p = plan(lens, 8, 32, 128, 16, 32, "workqueue")
    t = [2048, 100, 1, 0, 32]
    assert p.row_pages == t
    assert p.pages_per_split == 64  # ceil(2048 / 32), shared by the whole batch
    assert p.row_nsplit == [32, 2, 1, 0, 1]
    assert p.row_task_off == [0, 256, 272, 280, 280, 288]
    assert p.n_state_slots == len(p.tasks) == 288 and p.n_empty_slots == 0
    assert p.n_launches == 2
    assert p.merge_state_bytes == 2 * 288 * 4 * 130 * 4
    # Lexicographic (row, kv_head, split) order.
    assert p.tasks == sorted(p.tasks, key=lambda x: (x[0], x[1], x[2]))
    assert p.tasks[0] == (0, 0, 0, 0, 64) and p.tasks[31] == (0, 0, 31, 1984, 2048)
    assert p.tasks[256] == (1, 0, 0, 0, 64) and p.tasks[257] == (1, 0, 1, 64, 100)


def test_bucketed_closed_forms():
    lens = [300, 17, 300, 0]
    p = plan(lens, 2, 4, 64, 16, 4, "bucketed")
    # Buckets by ascending exact length: 0, 17, 300.
    assert [bk[0] for bk in p.buckets] == [0, 17, 300]
    assert p.buckets[0] == (0, 0, 1, 0, (3,))
    assert p.buckets[1] == (17, 2, 1, 2, (1,))      # T=2: pps=max(1,ceil(2/4))=1, 2 splits
    assert p.buckets[2] == (300, 19, 5, 4, (0, 2))  # T=19: pps=5, 4 splits
    assert p.n_launches == 6
    assert p.n_state_slots == 4 * 2 * 4
    assert p.n_empty_slots == 1 * 2 * 4 + 1 * 2 * 2
    assert p.row_nsplit == [4, 2, 4, 0]


def test_padded_closed_forms():
    # T = 19, 2, 19, 0, 5, 32 pages -> padded 32, 2, 32, 0, 8, 32.
    lens = [300, 17, 300, 0, 65, 512]
    p = plan(lens, 2, 4, 64, 16, 4, "padded")
    assert [bk[1] for bk in p.buckets] == [0, 2, 8, 32]
    assert p.buckets[0] == (-1, 0, 1, 0, (3,))
    assert p.buckets[1] == (-1, 2, 1, 2, (1,))        # pps = max(1, ceil(2/4)) = 1
    assert p.buckets[2] == (-1, 8, 2, 4, (4,))        # T=5 padded to 8: pps 2, row gets 3
    assert p.buckets[3] == (-1, 32, 8, 4, (0, 2, 5))  # pps 8: T=19 -> 3 splits, T=32 -> 4
    assert p.row_nsplit == [3, 2, 3, 0, 3, 4]
    assert p.n_launches == 8
    assert p.n_state_slots == 6 * 2 * 4
    # Row-local bounds: slots past each row's own split count are empty.
    assert p.n_empty_slots == 2 * sum(4 - ns for ns in p.row_nsplit)
    # The last split of a row stops at its real last page, not the padded one.
    assert (0, 1, 2, 16, 19) in p.tasks and (4, 0, 2, 4, 5) in p.tasks
    assert len(p.tasks) == 2 * sum(p.row_nsplit)


def test_padded_equals_bucketed_on_power_of_two_pages():
    """Rows whose page counts are distinct powers of two: padding is the identity."""
    lens = [16 * 1, 16 * 64, 16 * 8, 16 * 2048, 0]
    for s in [1, 3, 32]:
        a = plan(lens, 8, 32, 128, 16, s, "padded")
        b = plan(lens, 8, 32, 128, 16, s, "bucketed")
        assert a.tasks == b.tasks and a.row_nsplit == b.row_nsplit
        assert a.n_launches == b.n_launches and a.n_empty_slots == b.n_empty_slots
        assert [bk[1:] for bk in a.buckets] == [bk[1:] for bk in b.buckets]


def test_padded_brute_force_buckets():
    """Bucket of each row is the least power of two >= T_i; launches 2 x #distinct."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        lens = rng.integers(0, 5000, size=int(rng.integers(1, 12)))
        p = plan(lens, 1, 1, 64, 16, 8, "padded")
        want = {}
        for i, n in enumerate(lens):
            t = pages_of(n, 16)
            pad = next(q for q in [0] + [1 << k for k in range(20)] if q >= t)
            want.setdefault(pad, []).append(i)
        assert [(bk[1], bk[4]) for bk in p.buckets] == [(k, tuple(v)) for k, v in sorted(want.items())]
        assert p.n_launches == 2 * len(want)


def test_single_row_bucketed_equals_workqueue():
    for n in [1, 16, 17, 1000, 32768]:
        for s in [1, 4, 32]:
            a = plan([n], 8, 32, 128, 16, s, "workqueue")
            b = plan([n], 8, 32, 128, 16, s, "bucketed")
            assert a.tasks == b.tasks
            assert a.n_launches == b.n_launches == 2


def test_pages_launch_fanout_16_to_2():
    with open(os.path.join(GOLDEN, "launch_fanout.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(20260623)
    lens = np.concatenate([rng.integers(128, 2048, 4, endpoint=True),
                           rng.integers(16384, 32768, 4, endpoint=True)])
    assert len(set(lens.tolist())) == g["batch"]
    assert plan(lens, 8, 32, 128, 16, 32, "bucketed").n_launches == g[
        "exact_bucket_launches_per_step"]
    assert plan(lens, 8, 32, 128, 16, 32, "workqueue").n_launches == g[
        "compact_workqueue_launches_per_step"]


def test_compact_workqueue_cuts_merge_traffic_on_bimodal():
    """Direction only: short rows get fewer splits than in exact buckets."""
    rng = np.random.default_rng(20260622)
    lens = np.concatenate([rng.integers(128, 2048, 4, endpoint=True),
                           rng.integers(16384, 32768, 4, endpoint=True)])
    wq = plan(lens, 8, 32, 128, 16, 32, "workqueue")
    bk = plan(lens, 8, 32, 128, 16, 32, "bucketed")
    assert wq.merge_state_bytes < bk.merge_state_bytes


def test_nosplit_plan():
    p = plan([5, 0, 40], 2, 8, 64, 16, 32, "nosplit")
    assert p.tasks == [(0, 0, 0, 0, 1), (0, 1, 0, 0, 1), (2, 0, 0, 0, 3), (2, 1, 0, 0, 3)]
    assert p.n_launches == 1 and p.n_state_slots == 0 and p.merge_state_bytes == 0


def test_brute_force_granule_tiny():
    """Workqueue granule is the smallest page count that gives <= S splits to the longest row."""
    for t_max in range(0, 70):
        for s in range(1, 9):
            lens = [t_max * 4]
            p = plan(lens, 1, 1, 8, 4, s, "workqueue")
            best = next(g for g in range(1, max(t_max, 1) + 1) if -(-t_max // g) <= s)
            assert p.pages_per_split == best


def test_policy_first_match():
    rules = [
        (1, 1, 0, 1 << 30, "bucketed", 32),
        (2, 7, 0, 8192, "nosplit", 1),
        (2, 7, 8193, 1 << 30, "workqueue", 16),
        (8, 1 << 30, 0, 1 << 30, "workqueue", 32),
        (1, 1 << 30, 0, 1 << 30, "nosplit", 1),
    ]
    assert choose(rules, 1, 32768) == ("bucketed", 32)
    assert choose(rules, 4, 8192) == ("nosplit", 1)
    assert choose(rules, 4, 8193) == ("workqueue", 16)
    assert choose(rules, 7, 0) == ("nosplit", 1)
    assert choose(rules, 64, 5) == ("workqueue", 32)
    assert choose(rules[:1], 2, 5) is None
    assert choose([], 1, 1) is None
