"""Fit and check the learned cost model (an alternative to the threshold table).

    python -m paged_kv_gqa_block_amd.cost_fit fit     # CPU: from stored calibration timings
    python -m paged_kv_gqa_block_amd.cost_fit check   # GPU: held-out measurement

The PersistentKV summary pages leave a learned cost model as future work
("Conclusion").  Here the model is one linear function per path of the plan
features of include/pkv.h (pkv_cost_features: launches, KV and state
megabytes, per-CU critical pages, grid items, tasks), predicting the step time
in microseconds.  `fit` takes the calibration timings stored in
policy_table.json (every candidate path and split cap timed on seed 20260622
over the (B, N_max) grid), regenerates each cell's lengths from the same seed,
computes the features through the C ABI, and solves one least-squares problem
per path on the relative error (each row scaled by 1 / measured time),
with a small ridge term.  It also
reports how the model's choices compare with the measured best, in sample,
under 5-fold cross-validation over cells and leaving one batch size out.
`check` measures, on held-out seed 20260623, the model's choice beside the
table's choice and the four single paths, with interleaved repeats.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

from . import _lib, engine, traces
from .calibrate import CANDIDATES, FAMILIES, NOISE, SINGLE_PATHS, cell_spec, log

PATHS = ("bucketed", "workqueue", "nosplit", "padded")
RIDGE = 1e-3
NUM_CUS = 256  # MI355X compute units: feature f4 deals grid items over them


def sweep_problem(batch: int) -> _lib.pkv_problem:
    base = traces.get_spec(f"policy_b{batch}")
    return _lib.make_problem(batch, base.num_q_heads, base.num_kv_heads, base.head_dim,
                             base.page_size, 1 << 20, 32768 // base.page_size, base.dtype)


def samples_from_table(table: dict):
    """(cell, candidate, path, features, us) of every calibration timing."""
    out = []
    for key, cell in table["calibration"].items():
        b, cap = cell["batch"], cell["cap"]
        lens = traces.draw_lengths(cell_spec(b, cap),
                                   np.random.default_rng(table["calibration_seed"]))
        if int(lens.max()) != cell["n_max"]:
            raise RuntimeError(f"cell {key}: regenerated lengths differ from the measured ones")
        prob = sweep_problem(b)
        for cand, t in cell["times"].items():
            path, s = cand.split(":")
            f = _lib.pkv_cost_features(prob, lens, _lib.PATH_IDS[path], int(s),
                                       NUM_CUS).astype(np.float64)
            out.append((key, cand, path, f, t))
    return out


def fit(samples) -> dict:
    """Per path: w minimising sum ((w . f - t) / t)^2 + RIDGE * |w|^2.  The
    ridge term keeps the weights of features that the calibration grid cannot
    tell apart (tasks and grid items on the workqueue; state bytes and tasks
    at one group size) small instead of large and opposite."""
    w = {}
    for path in PATHS:
        rows = [(f, t) for _, _, p, f, t in samples if p == path]
        if not rows:
            continue
        x = np.array([f for f, _ in rows]) / np.array([t for _, t in rows])[:, None]
        w[path] = np.linalg.solve(x.T @ x + RIDGE * np.eye(x.shape[1]), x.T @ np.ones(len(rows)))
    return w


def choice_quality(w: dict, samples) -> dict:
    """Total time of the model's choice per cell against the measured best."""
    by = {}
    for key, cand, path, f, t in samples:
        by.setdefault(key, []).append((float(w[path] @ f), t, cand))
    chosen = best = 0.0
    worse = 0
    for lst in by.values():
        t_pick = min(lst)[1]
        t_best = min(v[1] for v in lst)
        chosen += t_pick
        best += t_best
        worse += t_pick > t_best * (1 + NOISE)
    return {"cells": len(by), "model_total_us": round(chosen, 2), "best_total_us": round(best, 2),
            "over_best": round(chosen / best - 1, 4), "cells_over_3pct": worse}


def cross_validate(samples) -> dict:
    cells = sorted({s[0] for s in samples})
    perm = np.random.default_rng(0).permutation(len(cells))
    folds = [{cells[i] for i in perm[k::5]} for k in range(5)]
    res = {}
    for name, groups in (("5fold", folds),
                         ("leave_one_batch_out",
                          [{c for c in cells if c.split(":")[0] == str(b)}
                           for b in traces.POLICY_BATCHES])):
        tot = {"model_total_us": 0.0, "best_total_us": 0.0, "cells_over_3pct": 0}
        for te in groups:
            q = choice_quality(fit([s for s in samples if s[0] not in te]),
                               [s for s in samples if s[0] in te])
            for k in tot:
                tot[k] += q[k]
        tot["over_best"] = round(tot["model_total_us"] / tot["best_total_us"] - 1, 4)
        tot["model_total_us"] = round(tot["model_total_us"], 2)
        tot["best_total_us"] = round(tot["best_total_us"], 2)
        res[name] = tot
    return res


def cmd_fit(args) -> int:
    with open(args.table) as f:
        table = json.load(f)
    samples = samples_from_table(table)
    w = fit(samples)
    rel = np.array([(float(w[p] @ f) - t) / t for _, _, p, f, t in samples])
    doc = {
        "about": "Learned cost model for MI355X: per-path linear model of the step time in "
                 "microseconds over the plan features of pkv_cost_features (include/pkv.h).",
        "trained_on": {"table": "policy_table.json calibration timings",
                       "seed": table["calibration_seed"], "samples": len(samples)},
        "num_cus": NUM_CUS,
        "ridge": RIDGE,
        "candidates": [{"path": p, "splits": s} for p, s in CANDIDATES],
        "weights": {p: [float(v) for v in w[p]] for p in PATHS},
        "fit": {"rms_relative_error": round(float(np.sqrt(np.mean(rel ** 2))), 4),
                "in_sample": choice_quality(w, samples), **cross_validate(samples)},
    }
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: {json.dumps(doc['fit'])}")
    return 0


def cmd_check(args) -> int:
    import torch

    from . import timing

    assert torch.cuda.is_available(), "the held-out check needs a GPU"
    with open(args.out) as f:
        doc = json.load(f)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != doc["num_cus"]:
        log(f"warning: the model was fitted for {doc['num_cus']} CUs, this device has {cus}")
    model = engine.load_cost_model(args.out)
    rules = engine.load_policy_table()
    held, totals = {}, {"model": 0.0, "table": 0.0, **{f"{p}:{s}": 0.0 for p, s in SINGLE_PATHS}}
    t0 = time.time()
    for family, pattern in FAMILIES:
        held[family] = {}
        for b in traces.POLICY_BATCHES:
            spec = traces.get_spec(pattern.format(b))
            w = traces.generate(spec, traces.HELD_OUT_SEED)
            lens = w["seq_lens"].numpy()
            m_path, m_s, pred = engine.choose_model(model, sweep_problem(b), lens)
            t_path, t_s = engine.choose(rules, b, int(lens.max()))
            configs = list(dict.fromkeys(list(SINGLE_PATHS) + [(t_path, t_s), (m_path, m_s)]))
            wd = engine.to_device(w)
            engine.validate_inputs(wd)
            views = timing.pool_copies(wd, 1.0, max_copies=8)
            times = timing.time_paths_interleaved(w, views, configs, "auto", args.steps,
                                                  args.warmup, repeats=7)
            t_model, t_table = times[f"{m_path}:{m_s}"], times[f"{t_path}:{t_s}"]
            best_single = min(times[f"{p}:{s}"] for p, s in SINGLE_PATHS)
            totals["model"] += t_model
            totals["table"] += t_table
            for p, s in SINGLE_PATHS:
                totals[f"{p}:{s}"] += times[f"{p}:{s}"]
            held[family][str(b)] = {
                "n_max": int(lens.max()), "model": f"{m_path}:{m_s}", "model_predicted_us":
                round(pred, 2), "table": f"{t_path}:{t_s}",
                "times": {k: round(v, 2) for k, v in times.items()},
                "model_over_best_single": round(t_model / best_single, 4),
                "table_over_best_single": round(t_table / best_single, 4)}
            log(f"  {spec.name}: model {m_path}:{m_s} {t_model:.2f} us (predicted {pred:.2f}), "
                f"table {t_path}:{t_s} {t_table:.2f} us, best single {best_single:.2f} us")
            del views, wd, w
            torch.cuda.empty_cache()
    doc["heldout"] = {"seed": traces.HELD_OUT_SEED, "device": torch.cuda.get_device_name(0),
                      "cells": held, "total_us": {k: round(v, 2) for k, v in totals.items()},
                      "seconds": round(time.time() - t0, 1)}
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: held-out totals {doc['heldout']['total_us']}")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("cmd", choices=("fit", "check"))
    ap.add_argument("--table", default=engine.POLICY_TABLE_PATH)
    ap.add_argument("--out", default=engine.COST_MODEL_PATH)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args(argv)
    return cmd_fit(args) if args.cmd == "fit" else cmd_check(args)


if __name__ == "__main__":
    sys.exit(main())
