"""Calibrate the adaptive path policy on one seed and check it on another.

    python -m paged_kv_gqa_block_amd.calibrate [--out policy_table.json]

The PersistentKV summary pages ("2. Calibrated adaptive policy"; "Results":
thresholds fixed on calibration seed 20260622, results on held-out seed
20260623) pick the execution path from the batch size B and the longest
context N_max with hand-calibrated thresholds.  Here the thresholds are
measured on this GPU.  Every candidate (exact buckets, the workqueue or
power-of-two padded buckets with a split cap of 8/16/32/64, or the
single-pass no-split kernel) is timed on the calibration seed for every
batch size of the sweep (64/8 heads, d=128, bf16) at a grid of longest
lengths H: one row of length H for B = 1 (a single row's work is set by its
length alone), and B rows drawn like the sweep families capped at H for
larger B (U[64,H] for H <= 2048, U[1024,H] above).  The candidates' timed
repeats are interleaved and spread over several placements of the buffers in
memory (time_cell); a candidate's time is the median of its repeats.  Each
interval between grid values gets the candidate that is good at both ends
(build_rules).  The table is then checked on the held-out seed on the two
families against the four fixed single paths (bucketed S=32, workqueue S=32,
no-split, padded S=32): per batch size the policy's time must be within the
measured noise band of the best one (heldout_cell).
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
# One row: its length alone sets the work, and below a few thousand tokens
# every candidate is launch-bound and within a few per cent of the others, so
# the grid is finer there.
SINGLE_ROW_LENGTHS = (128, 192, 256, 384, 512, 640, 768, 896, 1024, 1152, 1280, 1408, 1536,
                      1792, 2048, 2560, 3072, 4096, 6144, 8192, 12288, 16384, 24576, 32768)
CAPS = (256, 512, 1024, 1536, 2048, 4096, 8192, 16384, 32768)
FAMILIES = (("short", "policy_short_b{}"), ("long", "policy_b{}"))
NOISE = 0.03  # slowdown counted as a miss in the cost model's evaluation summaries
TRACE_CELLS = ("long", "bimodal", "zipf", "uniform", "tiny")
HELDOUT_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "policy_heldout.json")
MIN_BAND = 0.005  # floor of a cell's noise band (0.5 %)
MIN_REPEAT_US = 2000.0  # a timed repeat spans at least this much device time
ALLOCATIONS = 3  # placements of a cell's buffers in memory (time_cell)
ALLOC_PAD_BYTES = 37 << 20  # address shift between placements


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


def time_cell(w: dict, configs, steps: int, warmup: int, repeats: int,
              allocations: int = 1):
    """Interleaved timing of `configs` on one workload, on `allocations`
    fresh device copies of it.

    A launch-bound step's time moves by a few per cent with where its
    buffers land in memory (the paired ratio of two paths at B = 1 moved by
    up to 4 % between allocations while its spread within one allocation
    stayed under 1 %), so a cell's repeats are spread over several
    placements: before each copy, a pad of a different size shifts the
    allocator's addresses.  Each repeat spans at least MIN_REPEAT_US of
    device time.  Returns (median, repeats, host) per "path:splits" key --
    the median and the list over all repeats of all allocations, paired in
    order across keys -- and the steps per repeat."""
    keys = [f"{p}:{s}" for p, s in configs]
    runs = {k: [] for k in keys}
    host = {k: [] for k in keys}
    k_steps = None
    for a in range(allocations):
        pad = torch.empty(a * ALLOC_PAD_BYTES + 1, dtype=torch.uint8, device="cuda")
        wd = engine.to_device(w)
        engine.validate_inputs(wd)
        views = timing.pool_copies(wd, 1.0, max_copies=8)
        if k_steps is None:
            probe = timing.time_paths_interleaved(w, views, [("workqueue", w["spec"].splits)],
                                                  "auto", 10, warmup, repeats=1)
            k_steps = max(steps, int(np.ceil(MIN_REPEAT_US / max(1.0, min(probe.values())))))
        _, r, h = timing.time_paths_interleaved(w, views, configs, "auto", k_steps, warmup,
                                                repeats=repeats, return_runs=True)
        for k in keys:
            runs[k] += r[k]
            host[k].append(h[k])
        del views, wd, pad
        torch.cuda.empty_cache()
    med = {k: float(np.median(v)) for k, v in runs.items()}
    return med, runs, {k: float(np.median(v)) for k, v in host.items()}, k_steps


def measure(spec: traces.WorkloadSpec, seed: int, configs, steps: int, warmup: int,
            repeats: int = 7, allocations: int = 1):
    """Median step time of every configuration on one generated workload
    (time_cell: interleaved repeats on `allocations` placements)."""
    w = traces.generate(spec, seed)
    med, _, _, _ = time_cell(w, configs, steps, warmup, repeats, allocations)
    out = {}
    for path, s in configs:
        out[f"{path}:{s}"] = round(med[f"{path}:{s}"], 2)
        log(f"  {spec.name} seed={seed} {path:9s} S={s:2d}: {out[f'{path}:{s}']:9.2f} us/step")
    return int(w["seq_lens"].max()), out


def build_rules(calib: dict):
    """Rules from the calibration grid of every batch size.

    Lengths up to the first grid value take that value's fastest candidate.
    A length in (H_j, H_j+1] takes the candidate with the smallest worst-case
    slowdown against the fastest one at the two grid values that bracket it
    (ties: the smaller summed time): a length between grid values is served
    by a candidate that is good on both sides.  Lengths past the last grid
    value take its fastest candidate.  Equal neighbouring rules are merged."""
    def pick(times_list):
        def key(c):
            return (max(t[c] / min(t.values()) for t in times_list),
                    sum(t[c] for t in times_list))
        path, sp = min(times_list[0], key=key).split(":")
        return path, int(sp)

    rules = []
    batches = list(traces.POLICY_BATCHES)
    for k, b in enumerate(batches):
        b_hi = batches[k + 1] - 1 if k + 1 < len(batches) else (1 << 30)
        grid = grid_of(b)
        t = [calib[f"{b}:{n}"]["times"] for n in grid]
        cells = [(0, grid[0], pick([t[0]]))]
        cells += [(grid[j] + 1, grid[j + 1], pick([t[j], t[j + 1]]))
                  for j in range(len(grid) - 1)]
        cells.append((grid[-1] + 1, 1 << 30, pick([t[-1]])))
        first = len(rules)
        for lo, hi, (path, sp) in cells:
            if len(rules) > first and (rules[-1]["path"], rules[-1]["splits"]) == (path, sp):
                rules[-1]["nmax_hi"] = hi  # merge equal neighbours
            else:
                rules.append({"b_lo": b, "b_hi": b_hi, "nmax_lo": lo, "nmax_hi": hi,
                              "path": path, "splits": sp})
    return rules


def rel_iqr(xs) -> float:
    """Interquartile range over the median: the spread of one
    configuration's repeats."""
    q1, q2, q3 = np.percentile(np.asarray(xs, dtype=np.float64), [25, 50, 75])
    return float((q3 - q1) / q2) if q2 > 0 else 0.0


def heldout_cell(w: dict, path: str, s: int, steps: int, warmup: int, repeats: int,
                 allocations: int) -> dict:
    """One held-out cell: the policy's choice (path, s) against the four
    fixed single paths at the workload's own split cap.

    All of them are timed with time_cell.  The choice is compared with the
    single path of the lowest median through the ratios of their paired
    repeats (timed next to each other in every round, on every placement):
    the cell passes when the median ratio is at most 1 + band, the band
    being the interquartile range of those ratios (at least MIN_BAND) -- the
    measured spread of the comparison itself, placements included."""
    spec = w["spec"]
    singles = [(p, spec.splits if p != "nosplit" else 1) for p, _ in SINGLE_PATHS]
    configs = list(dict.fromkeys(singles + [(path, s)]))
    med, runs, host, k_steps = time_cell(w, configs, steps, warmup, repeats, allocations)
    key = f"{path}:{s}"
    best_key = min((f"{p}:{ss}" for p, ss in singles), key=lambda k: med[k])
    ratios = [a / b for a, b in zip(runs[key], runs[best_key])]
    ratio = float(np.median(ratios))
    q1, q3 = np.percentile(ratios, [25, 75])
    band = max(MIN_BAND, float(q3 - q1))
    return {"batch": spec.batch, "n_max": int(w["seq_lens"].max()),
            "steps_per_repeat": k_steps, "allocations": allocations,
            "policy": key, "best_single": best_key,
            "times_us": {k: round(v, 2) for k, v in med.items()},
            "single_us": {p: round(med[f"{p}:{ss}"], 2) for p, ss in singles},
            "repeats_us": {k: [round(x, 2) for x in v] for k, v in runs.items()},
            "spread": {k: round(rel_iqr(v), 4) for k, v in runs.items()},
            "host_enqueue_us": {k: round(v, 2) for k, v in host.items()},
            "band": round(band, 4), "policy_over_best_single": round(ratio, 4),
            "ok": ratio <= 1 + band}


def summarise(record: dict) -> tuple:
    """Whether every cell passed, and the policy's summed time against every
    single path's (the policy's sum must not exceed any of them)."""
    total_policy = sum(r["times_us"][r["policy"]] for r in record.values())
    total_single = {p: 0.0 for p, _ in SINGLE_PATHS}
    for r in record.values():
        for p, v in r["single_us"].items():
            total_single[p] += v
    totals = {"policy": round(total_policy, 2),
              **{k: round(v, 2) for k, v in total_single.items()}}
    sums_ok = all(total_policy <= v for v in total_single.values())
    return all(r["ok"] for r in record.values()), sums_ok, totals


def check_default(out_path: str, steps: int, warmup: int, repeats: int,
                  allocations: int) -> bool:
    """Held-out check of the engine's default policy (pkv_policy_default).

    Cells: both sweep families at every batch size and the trace workloads,
    all on the held-out seed; each cell is judged by heldout_cell, and over
    all cells the policy's summed time must not exceed any single path's
    sum."""
    rules = engine.load_policy_table()
    model = engine.load_cost_model()
    cells = [(pattern.format(b), family) for family, pattern in FAMILIES
             for b in traces.POLICY_BATCHES] + [(t, "trace") for t in TRACE_CELLS]
    record = {}
    for name, family in cells:
        w = traces.generate(traces.get_spec(name), traces.HELD_OUT_SEED)
        lens = w["seq_lens"].numpy()
        path, s = engine.choose_default(rules, model, engine.problem_from_workload(w), lens)
        rec = heldout_cell(w, path, s, steps, warmup, repeats, allocations)
        record[name] = {"family": family, **rec}
        log(f"  default policy {name}: {rec['policy']} {rec['times_us'][rec['policy']]:.2f} us, "
            f"best single {rec['best_single']} {rec['times_us'][rec['best_single']]:.2f} us, "
            f"ratio {rec['policy_over_best_single']:.4f} band {rec['band']:.4f} -> "
            f"{'ok' if rec['ok'] else 'SLOWER'}")
    ok_all, sums_ok, totals = summarise(record)
    doc = {
        "about": "Held-out check of the default policy (pkv_policy_default: calibrated table "
                 "for B = 1, learned cost model over the workqueue and no-split candidates "
                 "and the CU-balanced workqueue caps for B >= 2) against the four fixed "
                 "single paths.",
        "heldout_seed": traces.HELD_OUT_SEED,
        "device": torch.cuda.get_device_name(0),
        "repeats": repeats, "allocations": allocations, "min_band": MIN_BAND,
        "min_repeat_us": MIN_REPEAT_US,
        "cells": record,
        "total_us": totals,
        "sums_ok": sums_ok,
        "all_cells_ok": ok_all,
    }
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {out_path}: cells {'all ok' if ok_all else 'NOT all ok'}, sums "
        f"{'ok' if sums_ok else 'NOT ok'}; totals {totals}")
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
                         "B = 1, cost model with the balanced caps for B >= 2) and write "
                         "policy_heldout.json")
    ap.add_argument("--repeats", type=int, default=7,
                    help="timed repeats per placement")
    ap.add_argument("--allocations", type=int, default=ALLOCATIONS,
                    help="placements of each cell's buffers in memory")
    ap.add_argument("--batches", default=None,
                    help="with --rules-from: comma-separated batch sizes to measure again "
                         "(their cells replace the stored ones)")
    args = ap.parse_args(argv)
    assert torch.cuda.is_available(), "calibration needs a GPU"
    if args.check_default:
        out = args.out if args.out != engine.POLICY_TABLE_PATH else HELDOUT_PATH
        return 0 if check_default(out, args.steps, args.warmup, args.repeats,
                                  args.allocations) else 1
    t0 = time.time()
    calib, held = {}, {}
    if args.rules_from:
        with open(args.rules_from) as f:
            calib = json.load(f)["calibration"]
    if args.rules_from:
        again = [int(x) for x in args.batches.split(",")] if args.batches else []
        for b in again:  # cells measured again replace the stored ones
            calib = {k: v for k, v in calib.items() if v["batch"] != b}
    else:
        again = list(traces.POLICY_BATCHES)
    for b in again:
        for n in grid_of(b):
            n_max, times = measure(cell_spec(b, n), traces.CALIBRATION_SEED, CANDIDATES,
                                   args.steps, args.warmup, args.repeats, args.allocations)
            calib[f"{b}:{n}"] = {"batch": b, "cap": n, "n_max": n_max, "times": times}
    rules = build_rules(calib)
    rule_rows = [(r["b_lo"], r["b_hi"], r["nmax_lo"], r["nmax_hi"],
                  engine.PATH_IDS[r["path"]], r["splits"]) for r in rules]
    for family, pattern in FAMILIES:
        for b in traces.POLICY_BATCHES:
            w = traces.generate(traces.get_spec(pattern.format(b)), traces.HELD_OUT_SEED)
            path, s = engine.choose(rule_rows, b, int(w["seq_lens"].max()))
            rec = heldout_cell(w, path, s, args.steps, args.warmup, args.repeats,
                               args.allocations)
            held[f"{family}_b{b}"] = {"family": family, **rec}
            log(f"  held-out {w['spec'].name}: N_max {rec['n_max']} -> policy {rec['policy']} "
                f"{rec['times_us'][rec['policy']]:.2f} us, best single {rec['best_single']} "
                f"{rec['times_us'][rec['best_single']]:.2f} us, ratio "
                f"{rec['policy_over_best_single']:.4f} band {rec['band']:.4f} -> "
                f"{'ok' if rec['ok'] else 'SLOWER'}")
    ok_all, sums_ok, totals = summarise(held)
    doc = {
        "about": "Calibrated decode-path policy for MI355X (first matching rule wins).",
        "calibration_seed": traces.CALIBRATION_SEED,
        "heldout_seed": traces.HELD_OUT_SEED,
        "device": torch.cuda.get_device_name(0),
        "metric": "device us/step (split + merge launches, HIP graph replay), KV pools "
                  "rotated past the MALL",
        "repeats": args.repeats, "allocations": args.allocations, "min_band": MIN_BAND,
        "rules": rules,
        "calibration": calib,
        "heldout": held,
        "heldout_total_us": totals,
        "heldout_sums_ok": sums_ok,
        "heldout_ok": ok_all,
        "seconds": round(time.time() - t0, 1),
    }
    with open(args.out, "w") as f:
        json.dump(doc, f, indent=1)
    log(f"wrote {args.out}: held-out cells {'all ok' if ok_all else 'NOT all ok'}, sums "
        f"{'ok' if sums_ok else 'NOT ok'}; totals {totals}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
