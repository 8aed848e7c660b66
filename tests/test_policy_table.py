"""The calibrated policy table (CPU): coverage, C-ABI vs oracle, and the
recorded held-out check (calibrated on seed 20260622, checked on 20260623)."""
import json

import numpy as np

from oracle.policy import choose as oracle_choose
from paged_kv_gqa_block_amd import engine
from paged_kv_gqa_block_amd._lib import PATH_IDS, PATH_NAMES, pkv_policy


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


def test_recorded_heldout_check_passes():
    doc = _doc()
    assert doc["calibration_seed"] == 20260622 and doc["heldout_seed"] == 20260623
    assert doc["heldout_ok"] is True
    rules = engine.load_policy_table()
    for family in doc["heldout"].values():
        for b, rec in family.items():
            assert rec["ok"] and rec["policy_over_best_single"] <= 1 + doc["noise_band"]
            # The table reproduces the recorded choice for that (B, N_max).
            path, s = pkv_policy(rules, int(b), rec["n_max"])
            assert f"{PATH_NAMES[path]}:{s}" == rec["policy"]
    tot = doc["heldout_total_us"]
    assert tot["policy"] <= min(v for k, v in tot.items() if k != "policy")


def test_rules_use_known_paths():
    for r in _doc()["rules"]:
        assert r["path"] in PATH_IDS and 1 <= r["splits"] <= 64
        assert r["b_lo"] <= r["b_hi"] and r["nmax_lo"] <= r["nmax_hi"]
