"""The shipped learned cost model (CPU): its file is well formed, it was fitted
on the calibration seed's timings, the C choice equals the oracle's on the
sweep and trace workloads, and (once measured) the recorded held-out check."""
import json

import numpy as np
import pytest

import oracle
from paged_kv_gqa_block_amd import _lib, engine, traces


def _doc():
    with open(engine.COST_MODEL_PATH) as f:
        return json.load(f)


def test_model_file_is_well_formed():
    doc = _doc()
    assert doc["trained_on"]["seed"] == traces.CALIBRATION_SEED
    assert doc["num_cus"] == 256
    cands, weights, cus = engine.load_cost_model()
    assert len(cands) >= 4 and all(p in _lib.PATH_NAMES and s >= 1 for p, s in cands)
    assert set(weights) == {"mfma", "mfma_g16", "valu"}  # one per split-kernel variant
    for w in weights.values():
        assert w.shape == (4, _lib.PKV_COST_FEATURES) and np.isfinite(w).all()
        assert abs(w).max() < 1e3  # the ridge term keeps weights moderate
    for kernel, fit in doc["fit"].items():
        assert fit["rms_relative_error"] < 0.2, kernel
        assert fit["5fold"]["over_best"] < 0.05, kernel


@pytest.mark.parametrize("name", ["tiny", "long", "bimodal", "zipf", "uniform", "policy_b1",
                                  "policy_b8", "policy_b64", "policy_short_b16"])
def test_c_choice_equals_oracle_on_workloads(name):
    spec = traces.get_spec(name)
    lens = traces.draw_lengths(spec, np.random.default_rng(traces.HELD_OUT_SEED))
    cands, weights, cus = engine.load_cost_model()
    prob = _lib.make_problem(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                             spec.page_size, 1 << 20, 32768 // spec.page_size, spec.dtype)
    path, s, pred = engine.choose_model((cands, weights, cus), prob, lens)
    named = [(_lib.PATH_NAMES[p], ss) for p, ss in cands]
    w = weights[engine.split_kernel_of(prob)]
    ref = oracle.cost.choose(w.astype(np.float64), named, lens, spec.num_kv_heads,
                             spec.num_q_heads, spec.head_dim, spec.page_size, cus)
    assert (path, s) == ref[:2]
    assert pred == pytest.approx(ref[2], rel=1e-5)
    assert pred > 0


def test_recorded_heldout_check():
    doc = _doc()
    if "heldout" not in doc:
        pytest.skip("held-out measurement not recorded yet")
    h = doc["heldout"]
    assert h["seed"] == traces.HELD_OUT_SEED
    for family in h["cells"].values():
        for rec in family.values():
            assert rec["model"] in rec["times"] and rec["table"] in rec["times"]
            assert rec["model_over_best_single"] <= 1.10
    # Summed over the sweep families the model is no slower than any single path.
    totals = h["total_us"]
    singles = [v for k, v in totals.items() if ":" in k]
    assert totals["model"] <= min(singles)


def test_recorded_shape_checks():
    """Held-out timings of every candidate, the CU-balanced workqueue caps
    included, at four head shapes (cost_heldout_*.json, never used for
    fitting): the default policy's choices stay within 3 % of the best
    candidate at every shape, and in total are no slower than the model's
    choice among its listed candidates or the table's."""
    doc = _doc()
    checks = doc.get("shape_checks", {})
    if not checks:
        pytest.skip("shape checks not recorded yet")
    assert len(checks) >= 4
    for name, r in checks.items():
        assert r["seed"] == traces.HELD_OUT_SEED, name
        assert r["default_over_best"] <= 0.03, name
    total = {who: sum(r["total_us"][who] for r in checks.values())
             for who in ("default", "model", "table")}
    assert total["default"] <= min(total["model"], total["table"])



@pytest.mark.parametrize("name", ["cost_heldout_hq32_hkv2_f16.json",
                                  "cost_heldout_hq32_hkv8_f16_d64.json",
                                  "cost_heldout_hq32_hkv8_f16_skewed.json"])
def test_recorded_shape_checks_follow_from_the_stored_timings(name):
    """Scoring the stored held-out timings again (model and table choices
    through the C ABI) reproduces the recorded shape check exactly."""
    import os

    from paged_kv_gqa_block_amd import cost_fit

    doc = _doc()
    if name not in doc.get("shape_checks", {}):
        pytest.skip("shape check not recorded")
    path = os.path.join(os.path.dirname(engine.COST_MODEL_PATH), name)
    again = cost_fit.evaluate_file(path, engine.COST_MODEL_PATH)
    rec = doc["shape_checks"][name]
    assert again["total_us"] == rec["total_us"]
    assert again["cells_over_3pct"] == rec["cells_over_3pct"]
    assert again["default_over_best"] == rec["default_over_best"]
