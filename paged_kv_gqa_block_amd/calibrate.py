"""Calibrate the adaptive path policy on one seed and check it on another.

    python -m paged_kv_gqa_block_amd.calibrate [--out policy_table.json]

The PersistentKV summary pages ("2. Calibrated adaptive policy"; "Results":
thresholds fixed on calibration seed 20260622, results on held-out seed
20260623) pick the execution path from the batch size B and the longest
context N_max with hand-calibrated thresholds.  Here the thresholds are
measured on this GPU.  Every candidate (exact buckets, the workqueue or
power-of-two padded buckets with a split cap of 8/16/32/64, or the
single-pass no-split kernel) is timed on the
calibration seed for every batch size of the sweep (64/8 heads, d=128, bf16)
at a grid of longest lengths H: one row of length H for B = 1 (a single row's
work is set by its length alone), and B rows drawn like the sweep families
capped at H for larger B (U[64,H] for H <= 2048, U[1024,H] above), with the
candidates' timed repeats interleaved (median of 7).  The
fastest candidate becomes the rule of its (B range, N_max interval) cell,
with interval boundaries at the geometric midpoints between grid values.  The table is then
checked on the held-out seed on the two families against the four fixed
single paths (bucketed S=32, workqueue S=32, no-split, padded S=32): per batch size the
policy's time must be within the noise band of the best one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

from . import engine, timing, traces

CANDIDATES = ([("bucketed", s) for s in (8, 16, 32, 64)] +
              [("workqueue", s) for s in (8, 16, 32, 64)] +
              [("padded", s) for s in (8, 16, 32, 64)] + [("nosplit", 1)])
SINGLE_PATHS = (("bucketed", 32), ("workqueue", 32), ("nosplit", 1), ("padded", 32))
SINGLE_ROW_LENGTHS = (128, 256, 512, 768, 1024, 1536, 2048, 3072, 4096, 8192, 16384, 32768)
CAPS = (256, 512, 1024, 1536, 2048, 4096, 8192, 16384, 32768)
FAMILIES = (("short", "policy_short_b{}"), ("long", "policy_b{}"))
NOISE = 0.03  # run-to-run spread allowed when comparing to the best single path


def log(*a):
    print(*a, flush=True)


def cell_spec(batch: int, cap: int, num_q_heads: int | None = None,
              num_kv_heads: int | None = None, dtype: str | None = None,
              head_dim: int | None = None) -> traces.WorkloadSpec:
    """Calibration workload of batch size `batch` with longest length `cap`
    (head shape, head size and dtype of the sweep unless given; the lengths
    depend only on batch, cap and seed)."""
    base = traces.get_spec(f"policy_b{batch}")
    hq = num_q_heads or base.num_q_heads
    hkv = num_kv_heads or base.num_kv_heads
    dt = dtype or base.dtype
    d = head_dim or base.head_dim
    if batch == 1:
        return traces.WorkloadSpec(f"cal_b1_n{cap}", 1, hq, hkv, d, base.page_size,
                                   "fixed", base.splits, dt, fixed_len=cap)
    lo = 64 if cap <= 2048 else 1024
    return traces.WorkloadSpec(f"cal_b{batch}_h{cap}", batch, hq, hkv, d,
                               base.page_size, "uniform", base.splits, dt, lo=lo, hi=cap)


def grid_of(batch: int):
    return SINGLE_ROW_LENGTHS if batch == 1 else CAPS


def measure(spec: traces.WorkloadSpec, seed: int, configs, steps: int, warmup: int):
    name = spec.name
    w = traces.generate(spec, seed)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    views = timing.pool_copies(wd, 1.0, max_copies=8)
    times = timing.time_paths_interleaved(w, views, configs, "auto", steps, warmup, repeats=7)
    out = {}
    for path, s in configs:
        out[f"{path}:{s}"] = round(times[f"{path}:{s}"], 2)
        log(f"  {name} seed={seed} {path:9s} S={s:2d}: {out[f'{path}:{s}']:9.2f} us/step")
    n_max = int(w["seq_lens"].max())
    del views, wd, w
    torch.cuda.empty_cache()
    return n_max, out


def build_rules(calib: dict):
    def best(times):
        path, sp = min(times, key=times.get).split(":")
        return path, int(sp)

    rules = []
    batches = list(traces.POLICY_BATCHES)
    for k, b in enumerate(batches):
        b_hi = batches[k + 1] - 1 if k + 1 < len(batches) else (1 << 30)
        grid = grid_of(b)
        first = len(rules)
        for j, n in enumerate(grid):
            lo = 0 if j == 0 else int((grid[j - 1] * n) ** 0.5) + 1
            hi = (1 << 30) if j + 1 == len(grid) else int((n * grid[j + 1]) ** 0.5)
            path, sp = best(calib[f"{b}:{n}"]["times"])
            if len(rules) > first and (rules[-1]["path"], rules[-1]["splits"]) == (path, sp):
                rules[-1]["nmax_hi"] = hi  # merge equal neighbours
            else:
                rules.append({"b_lo": b, "b_hi": b_hi, "nmax_lo": lo, "nmax_hi": hi,
                              "path": path, "splits": sp})
    return rules


TRACE_CELLS = ("long", "bimodal", "zipf", "uniform", "tiny")
HELDOUT_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "policy_heldout.json")
MIN_BAND = 0.005  # floor of a cell's noise band (0.5 %)


def rel_iqr(xs) -> float:
    """Interquartile range over the median: the run-to-run spread of one
    configuration's repeats."""
    q1, q2, q3 = np.percentile(np.asarray(xs, dtype=np.float64), [25, 50, 75])
    return float((q3 - q1) / q2) if q2 > 0 else 0.0


def check_default(out_path: str, steps: int, warmup: int, repeats: int) -> bool:
    """Held-out check of the engine's default policy (pkv_policy_default).

    Cells: both sweep families at every batch size and the trace workloads,
    all on the held-out seed.  In each cell the default policy's choice and
    the four fixed single paths are timed with interleaved repeats.  The
    cell's noise band is the larger relative interquartile range of the
    policy's and the best single path's repeats (at least MIN_BAND): the
    policy passes the cell when its median is at most the best single
    path's median times (1 + band).  Over all cells its summed time must
    also not exceed any single path's sum.
    """
    rules = engine.load_policy_table()
    model = engine.load_cost_model()
    cells = [(pattern.format(b), family) for family, pattern in FAMILIES
             for b in traces.POLICY_BATCHES] + [(t, "trace") for t in TRACE_CELLS]
    record, ok_all = {}, True
    # Single paths at the workload's own split cap (32, or 4 for the tiny
    # workload), summed per path.
    total_policy, total_single = 0.0, {p: 0.0 for p, _ in SINGLE_PATHS}
    for name, family in cells:
        spec = traces.get_spec(name)
        w = traces.generate(spec, traces.HELD_OUT_SEED)
        lens = w["seq_lens"].numpy()
        path, s = engine.choose_default(rules, model, engine.problem_from_workload(w), lens)
        singles = [(p, spec.splits if p != "nosplit" else 1) for p, _ in SINGLE_PATHS]
        configs = list(dict.fromkeys(singles + [(path, s)]))
        wd = engine.to_device(w)
        engine.validate_inputs(wd)
        views = timing.pool_copies(wd, 1.0, max_copies=8)
        med, runs = timing.time_paths_interleaved(w, views, configs, "auto", steps, warmup,
                                                  repeats=repeats, return_runs=True)
        del views, wd
        torch.cuda.empty_cache()
        key = f"{path}:{s}"
        best_key = min((f"{p}:{ss}" for p, ss in singles), key=lambda k: med[k])
        band = max(MIN_BAND, rel_iqr(runs[key]), rel_iqr(runs[best_key]))
        ratio = med[key] / med[best_key]
        ok = ratio <= 1 + band
        ok_all &= ok
        total_policy += med[key]
        for p, ss in singles:
            total_single[p] += med[f"{p}:{ss}"]
        record[name] = {"family": family, "batch": spec.batch, "n_max": int(lens.max()),
                        "policy": key, "best_single": best_key,
                        "times_us": {k: round(v, 2) for k, v in med.items()},
                        "spread": {k: round(rel_iqr(v), 4) for k, v in runs.items()},
                        "band": round(band, 4), "policy_over_best_single": round(ratio, 4),
                        "ok": ok}
        log(f"  default policy {name}: {key} {med[key]:.2f} us, best single {best_key} "
            f"{med[best_key]:.2f} us, ratio {ratio:.4f} band {band:.4f} -> "
            f"{'ok' if ok else 'SLOWER'}")
    sums_ok = all(total_policy <= v for v in total_single.values())
    doc = {
        "about": "Held-out check of the default policy (pkv_policy_default: calibrated table "
                 "for B = 1, learned cost model over workqueue and no-split candidates for "
                 "B >= 2) against the four fixed single paths.",
        "heldout_seed": traces.HELD_OUT_SEED,
        "device": torch.cuda.get_device_name(0),
        "steps_per_repeat": steps, "repeats": repeats, "min_band": MIN_BAND,
        "cells": record,
        "total_us": {"policy": round(total_policy, 2),
                     **{k: round(v, 2) for k, v in total_single.items()}},
        "sums_ok": sums_ok,
        "all_cells_ok": ok_all,
    }
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {out_path}: cells {'all ok' if ok_all else 'NOT all ok'}, sums "
        f"{'ok' if sums_ok else 'NOT ok'}; totals {doc['total_us']}")
    return ok_all and sums_ok


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=engine.POLICY_TABLE_PATH)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rules-from", default=None,
                    help="reuse the calibration timings of this table; rebuild the rules "
                         "and rerun only the held-out check")
    ap.add_argument("--check-default", action="store_true",
                    help="only run the held-out check of the default policy (table for "
                         "B = 1, cost model for B >= 2) and write policy_heldout.json")
    ap.add_argument("--repeats", type=int, default=11)
    args = ap.parse_args(argv)
    assert torch.cuda.is_available(), "calibration needs a GPU"
    if args.check_default:
        out = args.out if args.out != engine.POLICY_TABLE_PATH else HELDOUT_PATH
        return 0 if check_default(out, args.steps, args.warmup, args.repeats) else 1
    t0 = time.time()
    calib, held = {}, {}
    if args.rules_from:
        with open(args.rules_from) as f:
            calib = json.load(f)["calibration"]
    for b in ([] if args.rules_from else traces.POLICY_BATCHES):
        for n in grid_of(b):
            n_max, times = measure(cell_spec(b, n), traces.CALIBRATION_SEED, CANDIDATES,
                                   args.steps, args.warmup)
            calib[f"{b}:{n}"] = {"batch": b, "cap": n, "n_max": n_max, "times": times}
    rules = build_rules(calib)
    rule_rows = [(r["b_lo"], r["b_hi"], r["nmax_lo"], r["nmax_hi"],
                  engine.PATH_IDS[r["path"]], r["splits"]) for r in rules]
    ok_all = True
    total_policy, total_single = 0.0, {f"{p}:{s}": 0.0 for p, s in SINGLE_PATHS}
    for family, pattern in FAMILIES:
        held[family] = {}
        for b in traces.POLICY_BATCHES:
            spec = traces.get_spec(pattern.format(b))
            lens = traces.draw_lengths(spec, np.random.default_rng(traces.HELD_OUT_SEED))
            path, s = engine.choose(rule_rows, b, int(lens.max()))
            configs = list(dict.fromkeys(list(SINGLE_PATHS) + [(path, s)]))
            n_max, times = measure(spec, traces.HELD_OUT_SEED, configs, args.steps, args.warmup)
            t_pol = times[f"{path}:{s}"]
            best_single = min(times[f"{p}:{ss}"] for p, ss in SINGLE_PATHS)
            ok = t_pol <= best_single * (1 + NOISE)
            ok_all &= ok
            total_policy += t_pol
            for p, ss in SINGLE_PATHS:
                total_single[f"{p}:{ss}"] += times[f"{p}:{ss}"]
            held[family][str(b)] = {"n_max": n_max, "policy": f"{path}:{s}", "times": times,
                                    "policy_over_best_single": round(t_pol / best_single, 4),
                                    "ok": ok}
            log(f"  held-out {spec.name}: N_max {n_max} -> policy {path}:{s} {t_pol:.2f} us, "
                f"best single {best_single:.2f} us -> {'ok' if ok else 'SLOWER'}")
    doc = {
        "about": "Calibrated decode-path policy for MI355X (first matching rule wins).",
        "calibration_seed": traces.CALIBRATION_SEED,
        "heldout_seed": traces.HELD_OUT_SEED,
        "noise_band": NOISE,
        "device": torch.cuda.get_device_name(0),
        "metric": "device us/step (split + merge launches), KV pools rotated past the MALL",
        "rules": rules,
        "calibration": calib,
        "heldout": held,
        "heldout_total_us": {"policy": round(total_policy, 2),
                             **{k: round(v, 2) for k, v in total_single.items()}},
        "heldout_ok": ok_all,
        "seconds": round(time.time() - t0, 1),
    }
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: held-out check {'passed' if ok_all else 'FAILED'}; "
        f"totals {doc['heldout_total_us']}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
