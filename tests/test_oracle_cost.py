"""Cost-model features and choice: the oracle against hand-computed values,
and the C entry points against the oracle (CPU only)."""
import math

import numpy as np
import pytest

from oracle import cost
from paged_kv_gqa_block_amd import _lib
from paged_kv_gqa_block_amd._lib import PATH_NAMES, PkvError

LENS = [300, 17, 300, 0]  # pages 19, 2, 19, 0


# Hand-computed plans of LENS with Hkv = 2, Hq = 4 (G = 2), d = 64, P = 16, S = 4
# and 4 CUs (each plan is also pinned by the planner closed-form tests):
#   workqueue: pps 5; tasks in grid order 5 5 5 4 | 5 5 5 4 | 2 | 2 | 5 5 5 4 | 5 5 5 4
#              -> CU sums 22 20 20 18, critical 22; 18 tasks; 2 launches; 18 slots
#   bucketed : launches for lengths 0 / 17 / 300; grids (row, head, slot):
#              0: eight empty slots -> 0; 17 (pps 1): 1 1 0 0 | 1 1 0 0 -> 2;
#              300 (pps 5): (5 5 5 4) x 4 -> CU sums 20 20 20 16 -> 20; total 22;
#              20 tasks; 6 launches; 32 slots
#   nosplit  : grid 19 19 2 2 19 19 0 0 -> CU sums 38 38 2 2 -> 38; 6 tasks; 8 items
#   padded   : pads 0 / 2 / 32; grids 0 -> 0; pad 2 (pps 1): 1 1 0 0 | 1 1 0 0 -> 2;
#              pad 32 (pps 8): (8 8 3 0) x 4 -> CU sums 32 32 12 0 -> 32; total 34;
#              16 tasks; 6 launches; 32 slots
#   largest task: workqueue 5, bucketed 5 (length 300), nosplit 19, padded 8 (pad 32)
KV_MB = 617 * 2 * 64 * 2 * 2 / 1e6
HAND = {
    "workqueue": [1, 2, KV_MB, 2 * 18 * 2 * 66 * 4 / 1e6, 22, 0.018, 0.018, 0.05],
    "bucketed": [1, 6, KV_MB, 2 * 32 * 2 * 66 * 4 / 1e6, 22, 0.032, 0.020, 0.05],
    "nosplit": [1, 1, KV_MB, 0, 38, 0.008, 0.006, 0.19],
    "padded": [1, 6, KV_MB, 2 * 32 * 2 * 66 * 4 / 1e6, 34, 0.032, 0.016, 0.08],
}


@pytest.mark.parametrize("path", sorted(HAND))
def test_oracle_features_match_hand_computation(path):
    f = cost.features(LENS, 2, 4, 64, 16, 4, path, 4)
    np.testing.assert_allclose(f, HAND[path], rtol=0, atol=1e-12)


@pytest.mark.parametrize("path", sorted(HAND))
def test_c_features_match_hand_computation(path):
    prob = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    got = _lib.pkv_cost_features(prob, LENS, _lib.PATH_IDS[path], 4, 4)
    np.testing.assert_allclose(got, HAND[path], rtol=1e-6, atol=1e-7)


def test_empty_batch_features_are_finite():
    f = cost.features([0, 0], 8, 32, 128, 16, 32, "workqueue", 256)
    assert f == [1.0, 1.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]


def test_oracle_choice_is_the_argmin():
    rng = np.random.default_rng(3)
    cands = [("workqueue", 8), ("workqueue", 32), ("bucketed", 32), ("padded", 16), ("nosplit", 1)]
    for _ in range(20):
        w = rng.normal(size=(4, cost.N_FEATURES))
        lens = rng.integers(0, 5000, size=int(rng.integers(1, 9)))
        path, s, y = cost.choose(w, cands, lens, 2, 8, 128, 16, 16)
        ys = [cost.predict_us(w, p, cost.features(lens, 2, 8, 128, 16, ss, p, 16))
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
            cus = int(rng.choice([1, 7, 256]))
            got = _lib.pkv_cost_features(prob, lens, path, s, cus)
            ref = cost.features(lens, hkv, hkv * g, 128, 16, s, PATH_NAMES[path], cus)
            np.testing.assert_allclose(got, ref, rtol=2e-7, atol=1e-6)


@pytest.mark.parametrize("seed", range(8))
def test_c_policy_model_matches_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    cands = [(p, s) for p in range(4) for s in (8, 16, 32, 64) if p != 2] + [(2, 1)]
    w = rng.normal(size=(4, cost.N_FEATURES))
    for _ in range(25):
        b = int(rng.integers(1, 65))
        lens = rng.integers(0, 32768, size=b, endpoint=True)
        prob = _lib.make_problem(b, 64, 8, 128, 16, 1 << 20, 2048)
        path, s, pred = _lib.pkv_policy_model(prob, cands, w.astype(np.float32), 256, lens)
        ys = [cost.predict_us(w.astype(np.float32), PATH_NAMES[p],
                              cost.features(lens, 8, 64, 128, 16, ss, PATH_NAMES[p], 256))
              for p, ss in cands]
        order = np.argsort(ys, kind="stable")
        scale = max(1.0, abs(ys[order[0]]))
        if ys[order[1]] - ys[order[0]] > 1e-5 * scale:  # a clear winner: both sides agree
            assert cands[order[0]] == (path, s)
        assert abs(pred - ys[cands.index((path, s))]) <= 1e-5 * max(1.0, abs(pred))


def test_policy_model_errors():
    prob = _lib.make_problem(2, 8, 2, 128, 16, 4096, 64)
    w = np.zeros((4, _lib.PKV_COST_FEATURES), np.float32)
    for cands, cus in (([(5, 8)], 256), ([(1, 0)], 256), ([(1, 8)], 0), ([(1, 8)], 1025)):
        with pytest.raises(PkvError) as e:
            _lib.pkv_policy_model(prob, cands, w, cus, [10, 20])
        assert e.value.status == _lib.PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_policy_model(prob, [(1, 8)], w, 256, [10, 64 * 16 + 1])
    assert e.value.status == _lib.PKV_ERANGE
    with pytest.raises(PkvError) as e:
        _lib.pkv_cost_features(prob, [10, 20], 4, 8, 256)
    assert e.value.status == _lib.PKV_EINVAL


# Hand-picked weights (rows: bucketed, workqueue, nosplit, padded) whose
# predictions on the HAND features above are worked out by hand:
#   bucketed  0 + 1 * 6 (launches) + 1 * 22 (critical pages)          = 28
#   workqueue 10 + 2 * 2 (launches) + 0.5 * 22 (critical pages)       = 25
#   nosplit   1 * 38 (critical pages)                                 = 38
#   padded    1 + 100 * 0.032 (grid items / 1000)                     = 4.2
HAND_W = [[0, 1, 0, 0, 1, 0, 0, 0],
          [10, 2, 0, 0, 0.5, 0, 0, 0],
          [0, 0, 0, 0, 1, 0, 0, 0],
          [1, 0, 0, 0, 0, 100, 0, 0]]
HAND_Y = {"bucketed": 28.0, "workqueue": 25.0, "nosplit": 38.0, "padded": 4.2}
HAND_CANDS = [("workqueue", 4), ("bucketed", 4), ("nosplit", 1), ("padded", 4)]


@pytest.mark.parametrize("path", sorted(HAND))
def test_predict_us_is_the_hand_computed_dot_product(path):
    assert abs(cost.predict_us(HAND_W, path, HAND[path]) - HAND_Y[path]) <= 1e-12


def test_choice_is_the_hand_worked_argmin():
    path, s, y = cost.choose(HAND_W, HAND_CANDS, LENS, 2, 4, 64, 16, 4)
    assert (path, s) == ("padded", 4) and abs(y - 4.2) <= 1e-12
    # The C entry point makes the same choice.
    prob = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    cands = [(_lib.PATH_IDS[p], ss) for p, ss in HAND_CANDS]
    w = np.asarray(HAND_W, dtype=np.float32)
    cp, cs, cy = _lib.pkv_policy_model(prob, cands, w, 4, LENS)
    assert (PATH_NAMES[cp], cs) == ("padded", 4) and abs(cy - 4.2) <= 1e-5


def test_choice_tie_goes_to_the_first_candidate():
    # bucketed now predicts 3 + 22 = 25, the workqueue's value; padded 100 + 3.2.
    w = [list(r) for r in HAND_W]
    w[0] = [3, 0, 0, 0, 1, 0, 0, 0]
    w[3] = [100, 0, 0, 0, 0, 100, 0, 0]
    assert cost.choose(w, HAND_CANDS, LENS, 2, 4, 64, 16, 4)[:2] == ("workqueue", 4)
    swapped = [HAND_CANDS[1], HAND_CANDS[0]] + HAND_CANDS[2:]
    assert cost.choose(w, swapped, LENS, 2, 4, 64, 16, 4)[:2] == ("bucketed", 4)
    prob = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    wf = np.asarray(w, dtype=np.float32)
    for order, want in ((HAND_CANDS, "workqueue"), (swapped, "bucketed")):
        cands = [(_lib.PATH_IDS[p], ss) for p, ss in order]
        assert PATH_NAMES[_lib.pkv_policy_model(prob, cands, wf, 4, LENS)[0]] == want


def test_default_policy_hand_worked():
    """One row: the table's rule for (1, N_1), whatever the model says; several
    rows: the model's argmin, whatever the table says."""
    from oracle import policy

    rules = [(1, 1, 0, 100, "nosplit", 1), (1, 1, 101, 1 << 30, "bucketed", 16),
             (2, 1 << 30, 0, 1 << 30, "nosplit", 1)]
    # One row of 300 tokens: rule 2 (bucketed, 16), although the model would
    # pick padded (HAND_W) for any lengths.
    assert policy.choose_default(rules, HAND_W, HAND_CANDS, [300], 2, 4, 64, 16, 4) == \
        ("bucketed", 16)
    # LENS (four rows): the model's hand-worked argmin, padded S=4, although
    # the table says nosplit for B >= 2.
    assert policy.choose_default(rules, HAND_W, HAND_CANDS, LENS, 2, 4, 64, 16, 4) == \
        ("padded", 4)
    # The C entry point agrees on both.
    cands = [(_lib.PATH_IDS[p], s) for p, s in HAND_CANDS]
    w = np.asarray(HAND_W, dtype=np.float32)
    crules = [r[:4] + (_lib.PATH_IDS[r[4]], r[5]) for r in rules]
    one = _lib.make_problem(1, 4, 2, 64, 16, 4096, 64)
    four = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    assert _lib.pkv_policy_default(crules, one, cands, w, 4, [300]) == (_lib.PKV_BUCKETED, 16)
    assert _lib.pkv_policy_default(crules, four, cands, w, 4, LENS) == (_lib.PKV_PADDED, 4)


# Workqueue task counts of LENS (pages 19, 2, 19, 0) with Hkv = 2, by cap S:
#   S=1: granule 19 -> 1 + 1 + 1 tasks per head -> 6;  S=2: granule 10 -> 2+1+2 -> 10;
#   S=3: granule 7 -> 3+1+3 -> 14;  S=4: granule 5 -> 4+1+4 -> 18;  S=5: granule 4 -> 5+1+5 -> 22
BALANCED_HAND = [  # (num_cus, per_cu, max_splits, cap)
    (4, 1, 64, 0),   # budget 4 < 6 tasks at S = 1
    (4, 2, 64, 1),   # budget 8
    (4, 3, 64, 2),   # budget 12
    (4, 5, 64, 4),   # budget 20: 18 <= 20 < 22
    (4, 5, 3, 3),    # the same budget, capped at 3
]


def test_balanced_splits_hand_counted():
    from oracle import policy

    prob = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    for cus, per_cu, smax, want in BALANCED_HAND:
        assert policy.balanced_splits(LENS, 2, 4, 64, 16, cus, per_cu, smax) == want
        assert _lib.pkv_balanced_splits(prob, LENS, cus, per_cu, smax) == want
    for bad in ((0, 1, 4), (4, 0, 4), (4, 65, 4), (4, 1, 0)):
        with pytest.raises(PkvError) as e:
            _lib.pkv_balanced_splits(prob, LENS, *bad)
        assert e.value.status == _lib.PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_balanced_splits(prob, [300, 17, 300, 64 * 16 + 1], 4, 1, 4)
    assert e.value.status == _lib.PKV_ERANGE


@pytest.mark.parametrize("seed", range(6))
def test_c_balanced_splits_matches_oracle(seed):
    from oracle import policy

    rng = np.random.default_rng(1700 + seed)
    for _ in range(6):
        b = int(rng.integers(1, 24))
        hkv = int(rng.choice([1, 2, 8]))
        lens = rng.integers(0, 8192, size=b, endpoint=True)
        lens[rng.random(b) < 0.2] = 0
        prob = _lib.make_problem(b, hkv * 4, hkv, 128, 16, 1 << 20, 512)
        cus, per_cu, smax = int(rng.choice([4, 64, 256])), int(rng.integers(1, 4)), 40
        assert _lib.pkv_balanced_splits(prob, lens, cus, per_cu, smax) == \
            policy.balanced_splits(lens, hkv, hkv * 4, 128, 16, cus, per_cu, smax)


def test_default_policy_takes_a_balanced_cap():
    """Weights that price the workqueue by its task count (1 µs per task) and
    every other path at 1000 µs: among HAND_CANDS the workqueue at S = 4 (18
    tasks) wins; the balanced cap for 2 tasks per CU on 4 CUs (S = 1, 6
    tasks) is cheaper still, and the default policy takes it.  The balanced
    cap for 1 task per CU does not exist (6 > 4 tasks at S = 1)."""
    from oracle import policy

    w = [[1000, 0, 0, 0, 0, 0, 0, 0], [0, 0, 0, 0, 0, 0, 1000, 0],
         [1000, 0, 0, 0, 0, 0, 0, 0], [1000, 0, 0, 0, 0, 0, 0, 0]]
    rules = [(1, 1 << 30, 0, 1 << 30, "nosplit", 1)]
    assert cost.choose(w, HAND_CANDS, LENS, 2, 4, 64, 16, 4)[:2] == ("workqueue", 4)
    assert policy.choose_default(rules, w, HAND_CANDS, LENS, 2, 4, 64, 16, 4) == \
        ("workqueue", 1)
    cands = [(_lib.PATH_IDS[p], s) for p, s in HAND_CANDS]
    crules = [r[:4] + (_lib.PATH_IDS[r[4]], r[5]) for r in rules]
    four = _lib.make_problem(4, 4, 2, 64, 16, 4096, 64)
    assert _lib.pkv_policy_default(crules, four, cands, np.asarray(w, np.float32), 4, LENS) == \
        (_lib.PKV_WORKQUEUE, 1)
    # With the workqueue at S = 1 listed, the listed candidate is scored and
    # the balanced cap adds nothing.
    listed = HAND_CANDS + [("workqueue", 1)]
    assert policy.choose_default(rules, w, listed, LENS, 2, 4, 64, 16, 4) == ("workqueue", 1)


@pytest.mark.parametrize("seed", range(6))
def test_c_default_policy_matches_oracle(seed):
    from oracle import policy
    from paged_kv_gqa_block_amd import engine

    rng = np.random.default_rng(1300 + seed)
    rules = engine.load_policy_table()
    cands_all, weights, cus = engine.load_cost_model()
    cands = [c for c in cands_all if c[0] in engine.DEFAULT_MODEL_PATHS]
    for _ in range(10):
        b = int(rng.choice([1, 1, 2, 5, 8, 33]))
        lens = rng.integers(0, 32768, size=b, endpoint=True)
        lens[0] = max(1, lens[0])
        prob = _lib.make_problem(b, 64, 8, 128, 16, 1 << 20, 2048, "bf16")
        w = weights[engine.split_kernel_of(prob)]
        got = _lib.pkv_policy_default(rules, prob, cands, w, cus, lens)
        orules = [r[:4] + (PATH_NAMES[r[4]], r[5]) for r in rules]
        ocands = [(PATH_NAMES[p], s) for p, s in cands]
        want = policy.choose_default(orules, w.astype(np.float64), ocands, lens, 8, 64, 128, 16,
                                     cus)
        if b == 1:
            assert (PATH_NAMES[got[0]], got[1]) == want
        else:  # the model's argmin; float32 (C) and float64 (oracle) may split a near tie
            caps = [policy.balanced_splits(lens, 8, 64, 128, 16, cus, k, 64) for k in (1, 2)]
            scored = ocands + [("workqueue", s) for s in caps if s > 0]
            assert (PATH_NAMES[got[0]], got[1]) in scored
            ys = {c: cost.predict_us(w, c[0], cost.features(lens, 8, 64, 128, 16, c[1], c[0],
                                                            cus)) for c in scored}
            best = min(ys.values())
            assert ys[(PATH_NAMES[got[0]], got[1])] <= best + 1e-4 * max(1.0, abs(best))
