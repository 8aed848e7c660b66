"""Cost-model features and choice: the oracle against hand-computed values,
and the C entry points against the oracle (CPU only)."""
import math

import numpy as np
import pytest

from oracle import cost
from paged_kv_gqa_block_amd import _lib
from paged_kv_gqa_block_amd._lib import PATH_NAMES, PkvError

LENS = [300, 17, 300, 0]  # pages 19, 2, 19, 0


def lg(x):
    return math.log2(x)


# Hand-computed plans of LENS with Hkv = 2, Hq = 4 (G = 2), d = 64, P = 16, S = 4
# (each also pinned by the planner closed-form tests):
#   bucketed : buckets 0 / 17 / 300; splits 0, 2, 4, 4 -> 20 tasks; 6 launches;
#              32 slots; longest task 5 pages (pps 5 for 19 pages)
#   workqueue: pps 5; splits 4, 1, 4, 0 -> 18 tasks; 2 launches; 18 slots
#   nosplit  : 3 non-empty rows x 2 heads = 6 tasks; 1 launch; 8 grid items;
#              longest task 19 pages
#   padded   : pads 32 / 2 / 32 / 0 -> 3 buckets; pps 8 and 1; splits 3, 2, 3
#              -> 16 tasks; 6 launches; 32 slots; longest task 8 pages
HAND = {
    "bucketed": [1, 2, lg(300), lg(617 / 4), 2, lg(20), 6, lg(32), lg(1 + 2 * 32 * 2 * 66 * 4),
                 lg(617 * 2 * 64 * 4), lg(5)],
    "workqueue": [1, 2, lg(300), lg(617 / 4), 2, lg(18), 2, lg(18), lg(1 + 2 * 18 * 2 * 66 * 4),
                  lg(617 * 2 * 64 * 4), lg(5)],
    "nosplit": [1, 2, lg(300), lg(617 / 4), 0, lg(6), 1, lg(8), 0, lg(617 * 2 * 64 * 4), lg(19)],
    "padded": [1, 2, lg(300), lg(617 / 4), 2, lg(16), 6, lg(32), lg(1 + 2 * 32 * 2 * 66 * 4),
               lg(617 * 2 * 64 * 4), lg(8)],
}


@pytest.mark.parametrize("path", sorted(HAND))
def test_oracle_features_match_hand_computation(path):
    f = cost.features(LENS, 2, 4, 64, 16, 4, path)
    np.testing.assert_allclose(f, HAND[path], rtol=0, atol=1e-12)


def test_empty_batch_features_are_finite():
    f = cost.features([0, 0], 8, 32, 128, 16, 32, "workqueue")
    assert all(math.isfinite(x) for x in f) and f[5] == 0 and f[6] == 1


def test_oracle_choice_is_the_argmin():
    rng = np.random.default_rng(3)
    cands = [("workqueue", 8), ("workqueue", 32), ("bucketed", 32), ("padded", 16), ("nosplit", 1)]
    for _ in range(20):
        w = rng.normal(size=(4, cost.N_FEATURES))
        lens = rng.integers(0, 5000, size=int(rng.integers(1, 9)))
        path, s, y = cost.choose(w, cands, lens, 2, 8, 128, 16)
        ys = [cost.predict_log2_us(w, p, cost.features(lens, 2, 8, 128, 16, ss, p))
              for p, ss in cands]
        assert y == min(ys) and cands[ys.index(min(ys))] == (path, s)


@pytest.mark.parametrize("seed", range(12))
def test_c_features_match_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    b = int(rng.integers(1, 40))
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8]))
    lens = rng.integers(0, 32768, size=b, endpoint=True)
    lens[rng.random(b) < 0.1] = 0
    prob = _lib.make_problem(b, hkv * g, hkv, 128, 16, 1 << 20, 2048)
    for path in range(4):
        for s in (1, 7, 32):
            got = _lib.pkv_cost_features(prob, lens, path, s)
            ref = cost.features(lens, hkv, hkv * g, 128, 16, s, PATH_NAMES[path])
            np.testing.assert_allclose(got, ref, rtol=2e-7, atol=2e-6)


@pytest.mark.parametrize("seed", range(8))
def test_c_policy_model_matches_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    cands = [(p, s) for p in range(4) for s in (8, 16, 32, 64) if p != 2] + [(2, 1)]
    w = rng.normal(scale=0.3, size=(4, cost.N_FEATURES))
    for _ in range(25):
        b = int(rng.integers(1, 65))
        lens = rng.integers(0, 32768, size=b, endpoint=True)
        prob = _lib.make_problem(b, 64, 8, 128, 16, 1 << 20, 2048)
        path, s, pred = _lib.pkv_policy_model(prob, cands, w.astype(np.float32), lens)
        ys = [cost.predict_log2_us(w.astype(np.float32), PATH_NAMES[p],
                                   cost.features(lens, 8, 64, 128, 16, ss, PATH_NAMES[p]))
              for p, ss in cands]
        order = np.argsort(ys, kind="stable")
        if ys[order[1]] - ys[order[0]] > 1e-4:  # a clear winner: both sides agree
            assert cands[order[0]] == (path, s)
        assert abs(math.log2(pred) - ys[cands.index((path, s))]) < 1e-4


def test_policy_model_errors():
    prob = _lib.make_problem(2, 8, 2, 128, 16, 4096, 64)
    w = np.zeros((4, _lib.PKV_COST_FEATURES), np.float32)
    for cands in ([(5, 8)], [(1, 0)]):
        with pytest.raises(PkvError) as e:
            _lib.pkv_policy_model(prob, cands, w, [10, 20])
        assert e.value.status == _lib.PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_policy_model(prob, [(1, 8)], w, [10, 64 * 16 + 1])
    assert e.value.status == _lib.PKV_ERANGE
    with pytest.raises(PkvError) as e:
        _lib.pkv_cost_features(prob, [10, 20], 4, 8)
    assert e.value.status == _lib.PKV_EINVAL
