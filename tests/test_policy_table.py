"""The calibrated policy table (CPU): coverage, C-ABI vs oracle, and the
recorded held-out check (calibrated on seed 20260622, checked on 20260623)."""
import json

import numpy as np

from oracle.policy import choose as oracle_choose
from paged_kv_gqa_block_amd import engine
from paged_kv_gqa_block_amd._lib import PATH_IDS, PATH_NAMES, make_problem, pkv_policy


def _doc():
    with open(engine.POLICY_TABLE_PATH) as f:
        return json.load(f)


def test_table_covers_every_batch_and_length():
    rules = engine.load_policy_table()
    rng = np.random.default_rng(0)
    for b in list(range(1, 130)) + [1000, 1 << 20]:
        for n in list(rng.integers(0, 40000, 20)) + [0, 1, 512, 2048, 2049, 32768, 1 << 29]:
            path, s = pkv_policy(rules, b, int(n))
            assert path in PATH_NAMES and s >= 1


def test_c_policy_equals_oracle_first_match():
    rules = engine.load_policy_table()
    rng = np.random.default_rng(1)
    for _ in range(2000):
        b, n = int(rng.integers(1, 100)), int(rng.integers(0, 40000))
        assert pkv_policy(rules, b, n) == oracle_choose(rules, b, n)


def _check_cell(rec, min_band, name):
    """A recorded held-out cell: recompute its paired-ratio statistic and band
    from the stored repeats and check the verdict."""
    ratios = [a / b for a, b in zip(rec["repeats_us"][rec["policy"]],
                                    rec["repeats_us"][rec["best_single"]])]
    assert len(ratios) == len(rec["repeats_us"][rec["best_single"]]) > 0, name
    band = max(min_band, float(np.subtract(*np.percentile(ratios, [75, 25]))))
    # The repeats are stored rounded to 0.01 us: a ratio moves by at most
    # 0.01 / (smallest repeat), a difference of two quantiles by twice that.
    tol = 0.02 / min(rec["repeats_us"][rec["best_single"]] + rec["repeats_us"][rec["policy"]])
    assert abs(band - rec["band"]) <= tol + 1e-4, name
    assert abs(float(np.median(ratios)) - rec["policy_over_best_single"]) <= tol + 1e-4, name
    # The best single path is one of the lowest median (the stored medians
    # are rounded to 0.01 us, so two paths with equal plans can tie).
    singles = rec["single_us"]
    assert singles[rec["best_single"].split(":")[0]] <= min(singles.values()) + 0.01, name
    assert rec["ok"] and float(np.median(ratios)) <= 1 + band, name


def test_recorded_heldout_check_passes():
    from paged_kv_gqa_block_amd import calibrate, traces

    doc = _doc()
    assert doc["calibration_seed"] == 20260622 and doc["heldout_seed"] == 20260623
    assert doc["heldout_ok"] is True and doc["heldout_sums_ok"] is True
    rules = engine.load_policy_table()
    want = {f"{f}_b{b}" for f, _ in calibrate.FAMILIES for b in traces.POLICY_BATCHES}
    assert set(doc["heldout"]) == want
    for name, rec in doc["heldout"].items():
        _check_cell(rec, doc["min_band"], name)
        # The table reproduces the recorded choice for that (B, N_max).
        path, s = pkv_policy(rules, rec["batch"], rec["n_max"])
        assert f"{PATH_NAMES[path]}:{s}" == rec["policy"]
    tot = doc["heldout_total_us"]
    assert tot["policy"] <= min(v for k, v in tot.items() if k != "policy")


def test_recorded_rules_follow_from_recorded_calibration():
    from paged_kv_gqa_block_amd import calibrate

    doc = _doc()
    assert calibrate.build_rules(doc["calibration"]) == doc["rules"]


def test_build_rules_brackets_each_interval():
    """Synthetic grid: the workqueue is 10 % faster than no-split everywhere
    except at the B = 1 grid values 1024 (no-split 1 % faster) and 1152
    (no-split 5 % faster).  Each interval between grid values takes the
    candidate with the smaller worst-case slowdown over its two ends."""
    from paged_kv_gqa_block_amd import calibrate, traces

    calib = {}
    for bb in traces.POLICY_BATCHES:
        for n in calibrate.grid_of(bb):
            t = {"workqueue:32": 10.0, "nosplit:1": 11.0}
            if bb == 1 and n == 1024:
                t = {"workqueue:32": 10.1, "nosplit:1": 10.0}
            if bb == 1 and n == 1152:
                t = {"workqueue:32": 10.5, "nosplit:1": 10.0}
            calib[f"{bb}:{n}"] = {"times": t}
    rules = [r for r in calibrate.build_rules(calib) if r["b_lo"] == 1]
    # (896, 1024]: workqueue (1 % at 1024) beats no-split (10 % at 896).
    # (1024, 1152]: no-split is fastest at both ends.
    # (1152, 1280]: workqueue (5 % at 1152) beats no-split (10 % at 1280).
    assert [(r["nmax_lo"], r["nmax_hi"], r["path"]) for r in rules] == [
        (0, 1024, "workqueue"), (1025, 1152, "nosplit"), (1153, 1 << 30, "workqueue")]
    assert rules[0]["b_hi"] == 1


def test_rules_use_known_paths():
    for r in _doc()["rules"]:
        assert r["path"] in PATH_IDS and 1 <= r["splits"] <= 64
        assert r["b_lo"] <= r["b_hi"] and r["nmax_lo"] <= r["nmax_hi"]


def test_recorded_default_policy_heldout_check():
    """The engine's default policy (table for B = 1, cost model with the
    CU-balanced workqueue caps for B >= 2) on
    the held-out seed, recorded by `calibrate --check-default`: every cell
    (both sweep families at every batch size, and the long, bimodal, zipf,
    uniform and tiny workloads) within its measured noise band of the best
    of the four fixed single paths, and the summed time below every single
    path's sum.  The recorded choices are still the ones the shipped table and
    model make."""
    from paged_kv_gqa_block_amd import calibrate, traces

    with open(calibrate.HELDOUT_PATH) as f:
        doc = json.load(f)
    assert doc["heldout_seed"] == traces.HELD_OUT_SEED
    cells = doc["cells"]
    want = {p.format(b) for _, p in calibrate.FAMILIES for b in traces.POLICY_BATCHES}
    assert want | set(calibrate.TRACE_CELLS) == set(cells)
    rules, model = engine.load_policy_table(), engine.load_cost_model()
    for name, rec in cells.items():
        _check_cell(rec, doc["min_band"], name)
        spec = traces.get_spec(name)
        lens = traces.draw_lengths(spec, np.random.default_rng(doc["heldout_seed"]))
        pages = max(1, int(-(-int(lens.max()) // spec.page_size)))
        prob = make_problem(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                            spec.page_size, 1 << 20, pages, spec.dtype)
        path, s = engine.choose_default(rules, model, prob, lens)
        assert f"{path}:{s}" == rec["policy"], name
    tot = doc["total_us"]
    assert doc["sums_ok"] and tot["policy"] <= min(v for k, v in tot.items() if k != "policy")
