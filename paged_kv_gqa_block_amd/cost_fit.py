"""Fit and check the learned cost model (an alternative to the threshold table).

    python -m paged_kv_gqa_block_amd.cost_fit measure --hq 32 --hkv 8 --dtype f16
                                                      # GPU: calibration timings, another shape
    python -m paged_kv_gqa_block_amd.cost_fit fit     # CPU: from stored calibration timings
    python -m paged_kv_gqa_block_amd.cost_fit check   # GPU: held-out measurement
    python -m paged_kv_gqa_block_amd.cost_fit measure --hq 32 --hkv 2 --seed 20260623
                                                      # GPU: held-out timings, another shape
    python -m paged_kv_gqa_block_amd.cost_fit evaluate cost_heldout_*.json
                                                      # CPU: the model's and the table's
                                                      #      choices on stored timings

The PersistentKV summary pages leave a learned cost model as future work
("Significado y Reivindicaciones" /
"Direcciones Futuras" on the es page).  Here the model is, for each split kernel (matrix-core or
vector-ALU) and each path, one linear function of the plan features of
include/pkv.h (pkv_cost_features: launches, KV and state megabytes, per-CU
critical pages, grid items, tasks), predicting the step time in
microseconds.  `fit` takes the calibration timings stored in
policy_table.json (every candidate path and split cap timed on seed 20260622
over the (B, N_max) grid), regenerates each cell's lengths from the same seed,
computes the features through the C ABI, and solves one least-squares problem
per (split kernel, path) on the relative error (each row scaled by 1 /
measured time), with a small ridge term.  It also reports how the model's
choices compare with the measured best, in sample, under 5-fold
cross-validation over cells, leaving one batch size out and leaving one head
shape out.  `measure` times the same candidates on the same (B, N_max) grid
and seed for another head shape, head size or dtype, with the table
calibration's protocol (interleaved repeats of at least 2 ms of device time,
on several placements of the buffers), and stores them beside
the table (cost_calib_*.json); `fit` uses every such file too.  `check` measures, on
held-out seed 20260623, the model's choice beside the table's choice and the
four single paths, with interleaved repeats: on the two sweep families and on
the trace workloads (another head shape and dtype).  `measure --seed
20260623` stores held-out timings of every candidate for a head shape
(cost_heldout_*.json, which `fit` does not read), and `evaluate` scores the
model's and the table's choices on such files: a check at head shapes and
head sizes the model was not trained on.
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import time

import numpy as np

from . import _lib, engine, traces
from .calibrate import (ALLOCATIONS, CANDIDATES, FAMILIES, NOISE, SINGLE_PATHS, cell_spec, grid_of,
                        log, measure, time_cell)

PATHS = ("bucketed", "workqueue", "nosplit", "padded")
RIDGE = 1e-3
NUM_CUS = 256  # MI355X compute units: feature f4 deals grid items over them


EXTRA_GLOB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_calib_*.json")
TRACE_WORKLOADS = ("long", "bimodal", "zipf", "uniform")


def sweep_problem(batch: int, shape: dict | None = None) -> _lib.pkv_problem:
    base = traces.get_spec(f"policy_b{batch}")
    shape = shape or {}
    return _lib.make_problem(batch, shape.get("num_q_heads", base.num_q_heads),
                             shape.get("num_kv_heads", base.num_kv_heads),
                             shape.get("head_dim", base.head_dim),
                             base.page_size, 1 << 20, 32768 // base.page_size,
                             shape.get("dtype", base.dtype))


def shape_tag(shape: dict | None) -> str:
    if not shape:
        return ""
    d = shape.get("head_dim", 128)
    return (f"{shape['num_q_heads']}/{shape['num_kv_heads']}/{shape['dtype']}"
            + (f"/d{d}" if d != 128 else "") + ":")


def shape_of(key: str) -> str:
    """The shape tag of a cell key ("" for the sweep's own shape)."""
    return ":".join(key.split(":")[:-2])


def kernel_of(key: str) -> str:
    """The split-kernel variant that ran a cell (engine.split_kernel_of): the
    vector-ALU kernel for d = 64 (head-size mark in the tag), else the
    matrix-core kernel for G <= 8 or its G = 16 variant."""
    tag = shape_of(key)
    if "/d" in tag:
        return "valu"
    if not tag:
        return "mfma"  # the sweep's own shape, 64/8
    hq, hkv = (int(x) for x in tag.split("/")[:2])
    return "mfma" if hq // hkv <= 8 else "mfma_g16"


KERNELS = ("mfma", "mfma_g16", "valu")


SKEWED = ("bimodal", "zipf")
SKEWED_BATCHES = (2, 4, 8, 16, 32)


def skewed_spec(dist: str, batch: int, shape: dict | None = None) -> traces.WorkloadSpec:
    """A batch of `batch` rows with the bimodal or Zipf length mix of the
    trace workloads, in the given head shape (the sweep's by default)."""
    base = traces.get_spec(dist)
    shape = shape or {}
    sweep = traces.get_spec("policy_b8")
    return traces.WorkloadSpec(f"cal_{dist}_b{batch}", batch,
                               shape.get("num_q_heads", sweep.num_q_heads),
                               shape.get("num_kv_heads", sweep.num_kv_heads),
                               shape.get("head_dim", sweep.head_dim), base.page_size,
                               base.lengths, base.splits, shape.get("dtype", sweep.dtype),
                               lo=base.lo, hi=base.hi)


def spec_of_cell(cell: dict, shape: dict | None = None) -> traces.WorkloadSpec:
    """The workload a stored calibration cell timed: a sweep cell (batch,
    longest length) or a skewed cell (batch, length mix)."""
    if "dist" in cell:
        return skewed_spec(cell["dist"], cell["batch"], shape)
    return cell_spec(cell["batch"], cell["cap"])


def samples_from_table(table: dict, shape: dict | None = None):
    """(cell, candidate, path, features, us) of every calibration timing."""
    out = []
    tag = shape_tag(shape)
    for key, cell in table["calibration"].items():
        b = cell["batch"]
        lens = traces.draw_lengths(spec_of_cell(cell, shape),
                                   np.random.default_rng(table["calibration_seed"]))
        if int(lens.max()) != cell["n_max"]:
            raise RuntimeError(f"cell {key}: regenerated lengths differ from the measured ones")
        prob = sweep_problem(b, shape)
        key = tag + key
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
                          [{c for c in cells if c.split(":")[-2] == str(b)}
                           for b in traces.POLICY_BATCHES]),
                         ("leave_one_shape_out",
                          [{c for c in cells if shape_of(c) == t}
                           for t in sorted({shape_of(c) for c in cells})])):
        if any(not g for g in groups) or len(groups) < 2:
            continue
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


SWEEP_SHAPE = {"num_q_heads": 64, "num_kv_heads": 8, "dtype": "bf16", "head_dim": 128}


def all_samples(table_path: str):
    """Every calibration timing: the cost_calib_*.json files, and the policy
    table's own timings unless one of those files covers the table's sweep
    shape (then the table's cells would be counted twice)."""
    with open(table_path) as f:
        table = json.load(f)
    extras = []
    for path in sorted(glob.glob(EXTRA_GLOB)):
        with open(path) as f:
            extras.append((os.path.basename(path), json.load(f)))
    samples, sources = [], []
    if not any(doc["shape"] == SWEEP_SHAPE for _, doc in extras):
        samples, sources = samples_from_table(table), ["policy_table.json"]
    for name, doc in extras:
        samples += samples_from_table(doc, doc["shape"])
        sources.append(name)
    return table, samples, sources


def balanced_candidates(prob, lens):
    """The CU-balanced workqueue caps that the default policy adds to the
    model's candidates (pkv_policy_default), when not among them."""
    caps = [s for p, s in CANDIDATES if p == "workqueue"]
    out = []
    for per_cu in (1, 2):
        s = _lib.pkv_balanced_splits(prob, lens, NUM_CUS, per_cu, max(caps))
        if s > 0 and ("workqueue", s) not in list(CANDIDATES) + out:
            out.append(("workqueue", s))
    return out


def cmd_measure(args) -> int:
    import torch

    assert torch.cuda.is_available(), "measuring needs a GPU"
    shape = {"num_q_heads": args.hq, "num_kv_heads": args.hkv, "dtype": args.dtype,
             "head_dim": args.d}
    calib = {}
    t0 = time.time()
    if args.skewed:
        for dist in SKEWED:
            for b in SKEWED_BATCHES:
                spec = skewed_spec(dist, b, shape)
                lens = traces.draw_lengths(spec, np.random.default_rng(args.seed))
                configs = list(CANDIDATES) + balanced_candidates(sweep_problem(b, shape), lens)
                n_max, times = measure(spec, args.seed, configs, args.steps, args.warmup,
                                       args.repeats, args.allocations)
                calib[f"{b}:{dist}"] = {"batch": b, "dist": dist, "n_max": n_max, "times": times}
            log(f"  {dist}: {len(SKEWED_BATCHES)} cells timed ({time.time() - t0:.0f} s so far)")
    for b in ([] if args.skewed else traces.POLICY_BATCHES):
        for n in grid_of(b):
            spec = cell_spec(b, n, args.hq, args.hkv, args.dtype, args.d)
            lens = traces.draw_lengths(spec, np.random.default_rng(args.seed))
            configs = list(CANDIDATES) + balanced_candidates(sweep_problem(b, shape), lens)
            n_max, times = measure(spec, args.seed, configs, args.steps, args.warmup,
                                   args.repeats, args.allocations)
            calib[f"{b}:{n}"] = {"batch": b, "cap": n, "n_max": n_max, "times": times}
        log(f"  B={b}: {len(grid_of(b))} cells timed ({time.time() - t0:.0f} s so far)")
    held_out = args.seed != traces.CALIBRATION_SEED
    doc = {"about": ("Held-out timings of every candidate path on the (B, N_max) grid for one "
                     "head shape, used to check the cost model (not to fit it)." if held_out else
                     "Calibration timings of every candidate path on the (B, N_max) grid for "
                     "one head shape, used to fit the cost model."),
           "shape": shape, "calibration_seed": args.seed,
           "device": torch.cuda.get_device_name(0), "repeats": args.repeats,
           "allocations": args.allocations, "calibration": calib,
           "seconds": round(time.time() - t0, 1)}
    stem = (f"hq{args.hq}_hkv{args.hkv}_{args.dtype}" + (f"_d{args.d}" if args.d != 128 else "")
            + ("_skewed" if args.skewed else ""))
    name = f"cost_heldout_{stem}.json" if held_out else f"cost_calib_{stem}.json"
    out = args.out if args.out != engine.COST_MODEL_PATH else os.path.join(
        os.path.dirname(engine.COST_MODEL_PATH), name)
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {out}")
    return 0


def cmd_fit(args) -> int:
    table, samples, sources = all_samples(args.table)
    weights, stats = {}, {}
    for kernel in KERNELS:  # one model per split kernel: their costs per page differ
        ss = [s for s in samples if kernel_of(s[0]) == kernel]
        if not ss:
            continue
        w = fit(ss)
        rel = np.array([(float(w[p] @ f) - t) / t for _, _, p, f, t in ss])
        weights[kernel] = {p: [float(v) for v in w[p]] for p in PATHS}
        stats[kernel] = {"samples": len(ss), "shapes": sorted({shape_of(s[0]) or "sweep"
                                                               for s in ss}),
                         "rms_relative_error": round(float(np.sqrt(np.mean(rel ** 2))), 4),
                         "in_sample": choice_quality(w, ss), **cross_validate(ss)}
    doc = {
        "about": "Learned cost model for MI355X: per split kernel and per path, a linear model "
                 "of the step time in microseconds over the plan features of "
                 "pkv_cost_features (include/pkv.h).",
        "trained_on": {"files": sources, "seed": table["calibration_seed"],
                       "samples": len(samples)},
        "num_cus": NUM_CUS,
        "ridge": RIDGE,
        "candidates": [{"path": p, "splits": s} for p, s in CANDIDATES],
        "weights": weights,
        "fit": stats,
    }
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: {json.dumps(doc['fit'])}")
    return 0


def cmd_check(args) -> int:
    import torch

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
            times, _, _, _ = time_cell(w, configs, args.steps, args.warmup, args.repeats,
                                       args.allocations)
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
    held["traces"] = {}
    for name in TRACE_WORKLOADS:
        spec = traces.get_spec(name)
        w = traces.generate(spec, traces.HELD_OUT_SEED)
        lens = w["seq_lens"].numpy()
        m_path, m_s, pred = engine.choose_model(model, engine.problem_from_workload(w), lens)
        t_path, t_s = engine.choose(rules, spec.batch, int(lens.max()))
        singles = [(p, (1 if p == "nosplit" else spec.splits)) for p, _ in SINGLE_PATHS]
        configs = list(dict.fromkeys(singles + [(t_path, t_s), (m_path, m_s)]))
        times, _, _, _ = time_cell(w, configs, args.steps, args.warmup, args.repeats,
                                   args.allocations)
        t_model, t_table = times[f"{m_path}:{m_s}"], times[f"{t_path}:{t_s}"]
        best_single = min(times[f"{p}:{s}"] for p, s in singles)
        held["traces"][name] = {
            "n_max": int(lens.max()), "model": f"{m_path}:{m_s}", "model_predicted_us":
            round(pred, 2), "table": f"{t_path}:{t_s}",
            "times": {k: round(v, 2) for k, v in times.items()},
            "model_over_best_single": round(t_model / best_single, 4),
            "table_over_best_single": round(t_table / best_single, 4)}
        log(f"  {name}: model {m_path}:{m_s} {t_model:.2f} us (predicted {pred:.2f}), "
            f"table {t_path}:{t_s} {t_table:.2f} us, best single {best_single:.2f} us")
    doc["heldout"] = {"seed": traces.HELD_OUT_SEED, "device": torch.cuda.get_device_name(0),
                      "repeats": args.repeats, "allocations": args.allocations,
                      "cells": held, "total_us": {k: round(v, 2) for k, v in totals.items()},
                      "seconds": round(time.time() - t0, 1)}
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: held-out totals {doc['heldout']['total_us']}")
    return 0


def evaluate_file(path: str, model_path: str) -> dict:
    """The model's, the table's and the default policy's choices against the
    best candidate and the best single path, on the stored timings of one
    file (any shape, any seed)."""
    with open(path) as f:
        doc = json.load(f)
    shape = doc["shape"]
    model = engine.load_cost_model(model_path)
    rules = engine.load_policy_table()
    tot = {"model": 0.0, "table": 0.0, "default": 0.0, "best": 0.0,
           **{f"{p}:{s}": 0.0 for p, s in SINGLE_PATHS}}
    worse = {"model": 0, "table": 0, "default": 0}
    for cell in doc["calibration"].values():
        b, times = cell["batch"], cell["times"]
        lens = traces.draw_lengths(spec_of_cell(cell, shape),
                                   np.random.default_rng(doc["calibration_seed"]))
        if int(lens.max()) != cell["n_max"]:
            raise RuntimeError(f"{path}: regenerated lengths differ from the measured ones")
        m_path, m_s, _ = engine.choose_model(model, sweep_problem(b, shape), lens)
        t_path, t_s = engine.choose(rules, b, int(lens.max()))
        d_path, d_s = engine.choose_default(rules, model, sweep_problem(b, shape), lens)
        best = min(times.values())
        for who, key in (("model", f"{m_path}:{m_s}"), ("table", f"{t_path}:{t_s}"),
                         ("default", f"{d_path}:{d_s}")):
            tot[who] += times[key]
            worse[who] += times[key] > best * (1 + NOISE)
        tot["best"] += best
        for p, s in SINGLE_PATHS:
            tot[f"{p}:{s}"] += times[f"{p}:{s}"]
    return {"file": os.path.basename(path), "shape": shape, "seed": doc["calibration_seed"],
            "cells": len(doc["calibration"]),
            "total_us": {k: round(v, 2) for k, v in tot.items()},
            "model_over_best": round(tot["model"] / tot["best"] - 1, 4),
            "table_over_best": round(tot["table"] / tot["best"] - 1, 4),
            "default_over_best": round(tot["default"] / tot["best"] - 1, 4),
            "cells_over_3pct": worse}


def cmd_evaluate(args) -> int:
    with open(args.out) as f:
        doc = json.load(f)
    res = [evaluate_file(p, args.out) for p in args.files]
    for r in res:
        log(json.dumps(r))
    doc["shape_checks"] = {r["file"]: r for r in res}
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("cmd", choices=("measure", "fit", "check", "evaluate"))
    ap.add_argument("files", nargs="*", help="evaluate: timing files (cost_*.json)")
    ap.add_argument("--hq", type=int, default=32)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--seed", type=int, default=traces.CALIBRATION_SEED)
    ap.add_argument("--dtype", default="f16")
    ap.add_argument("--table", default=engine.POLICY_TABLE_PATH)
    ap.add_argument("--out", default=engine.COST_MODEL_PATH)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=7,
                    help="measure, check: interleaved timed repeats per placement")
    ap.add_argument("--allocations", type=int, default=ALLOCATIONS,
                    help="measure, check: placements of each cell's buffers in memory")
    ap.add_argument("--skewed", action="store_true",
                    help="measure: bimodal and Zipf length mixes at B in "
                         f"{SKEWED_BATCHES} instead of the (B, N_max) grid")
    args = ap.parse_args(argv)
    return {"measure": cmd_measure, "fit": cmd_fit, "check": cmd_check,
            "evaluate": cmd_evaluate}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
