"""Decode-attention benchmark: µs per decode step and achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long]
                    [--path bucketed|workqueue|nosplit|padded|policy|model|default|device|selfplan]
                    [--kernel auto|valu|mfma] [--launch graph|eager]

One step is the engine's device work for one decode step of one layer: the
split kernel launch(es) and the merge launch(es) (or the single no-split
launch), with the plan already resident on the GPU.  Inputs are generated
(seeded, synthetic) and copied to HBM before timing.  To keep the 256 MB
Infinity Cache from serving K/V, every step reads a different copy of the KV
pools (as consecutive layers of a model would), with enough copies to exceed
1 GiB.  By default the K timed steps are launched eagerly, back to back (the
host enqueues a kernel in a few microseconds, well under the device time of
these steps); with --launch graph they are captured once in a HIP graph,
launched once untimed and then replayed.  The line also reports the same K
steps launched the other way (on these device-bound steps the two agree
within about 1 us per step; the short launch-bound steps of the policy sweep
are where graph replay pays).  For the long and bimodal workloads the line
carries both target workloads' figures in `targets`, each with the step time
of the engine's default policy (its own path and split cap) beside it.

Printed JSON line: value = real-KV bytes (sum N_i * Hkv * d * 2 * 2) divided by
the device step time measured with HIP events on the launch stream.  The
roofline object reports the split kernel alone, against the 8 TB/s HBM peak
and, beside it, against a read-only probe kernel that streams exactly the
same pages (the rate this access pattern reaches on the device);
cpu_baseline times the fp64 CPU oracle on the same generated inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step and achieved HBM GB/s (% of peak), paged GQA"
HBM_PEAK_GBS = 8000.0
# Counter-based HBM traffic of the split kernel per workload (rocprofv3
# FETCH_SIZE + WRITE_SIZE runs, scaled against a copy kernel); reported only
# while the device sources (every file under csrc/) still hash to the value
# recorded with it.
TRAFFIC_PROFILES = {"long": "profiles/split_mfma_long_b1_n32768_traffic.txt",
                    "bimodal": "profiles/split_mfma_bimodal_b8_traffic.txt",
                    "zipf": "profiles/split_mfma_zipf_b8_traffic.txt",
                    "uniform": "profiles/split_mfma_uniform_b8_traffic.txt",
                    "policy_b64": "profiles/split_mfma_policy_b64_traffic.txt"}
DEFAULT_PATH = {"tiny": "workqueue", "long": "bucketed", "bimodal": "workqueue",
                "zipf": "workqueue", "uniform": "workqueue"}


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default="long")
    p.add_argument("--path", default=None)
    p.add_argument("--splits", type=int, default=None)
    p.add_argument("--kernel", default="auto")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--copies-gib", type=float, default=1.0,
                   help="total size of the rotated KV pool copies")
    p.add_argument("--launch", choices=("graph", "eager"), default="eager",
                   help="graph: the K timed steps are captured once in a HIP "
                        "graph, launched once untimed, then replayed -- device time, as a "
                        "serving loop that replays its decode graph sees it; eager (the "
                        "default): one host "
                        "call per kernel")
    p.add_argument("--no-targets", action="store_true",
                   help="skip the second target workload's figures")
    p.add_argument("--all", action="store_true",
                   help="instead of the single contract line, print one JSON line per "
                        "(workload, path) for every workload, each with a short CPU-oracle "
                        "sample")
    return p.parse_args(argv)


def describe(spec, path, splits, lens):
    return (f"{spec.name}: B={spec.batch} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} "
            f"d={spec.head_dim} P={spec.page_size} S={splits} {spec.dtype} path={path} "
            f"N={'/'.join(str(int(n)) for n in lens) if len(lens) <= 8 else f'{len(lens)} rows'}")


def kernel_source_hash() -> str:
    """First 16 hex digits of the sha256 over every file under csrc/, in name
    order, each as its name followed by its bytes."""
    import hashlib

    csrc = os.path.join(ROOT, "paged_kv_gqa_block_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        path = os.path.join(csrc, name)
        if os.path.isfile(path):
            h.update(name.encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(config: str, kernel_used: str, path: str, splits: int, seed: int):
    """Traffic bytes per split launch from profiles/, or None if absent, stale or
    taken in another launch configuration (the profiles use the workload's
    default path and split cap, seed 20260623)."""
    from paged_kv_gqa_block_amd import traces

    rel = TRAFFIC_PROFILES.get(config)
    if rel is None or kernel_used != "mfma":
        return None
    if (path != DEFAULT_PATH.get(config, "workqueue") or splits != traces.get_spec(config).splits
            or seed != traces.HELD_OUT_SEED):
        return None
    try:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines()
                  if line.startswith(("kernel_source_sha256_16:", "traffic_bytes_per_launch:")))
    if fields.get("kernel_source_sha256_16", "").split()[0:1] != [kernel_source_hash()]:
        return None
    return int(fields["traffic_bytes_per_launch"].strip())


def host_cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s):
    import numpy as np

    import oracle
    from paged_kv_gqa_block_amd import traces

    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    a = traces.oracle_arrays(w)
    spec = w["spec"]
    lens = a["seq_lens"]
    rows = list(range(spec.batch))
    kv_row_bytes = [int(n) * spec.num_kv_heads * spec.head_dim * 2 * 2 for n in lens]
    done_bytes, reps = 0, 0
    t0 = time.perf_counter()
    # Whole decode steps while within budget; at least one row.
    while True:
        for i in rows:
            oracle.attention(a["q"], a["k_pool"], a["v_pool"], a["block_table"], lens,
                             a["scale"], a["page_size"], a["dtype"], rows=[i])
            done_bytes += kv_row_bytes[i]
            if time.perf_counter() - t0 > budget_s:
                break
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"fp64 numpy oracle on the same {spec.name} inputs: {reps} pass(es) over "
                      f"rows in order, {done_bytes / 1e6:.1f} MB of real KV in {dt:.1f} s "
                      f"({os.cpu_count()} host cpus visible)",
            "us_per_step_equiv": dt / max(done_bytes, 1) * sum(kv_row_bytes) * 1e6}


ALL_CONFIGS = ("tiny", "long", "bimodal", "zipf", "uniform") + tuple(
    f"policy_b{b}" for b in (1, 2, 4, 8, 16, 32, 64))


def run_all(args) -> int:
    """Every workload x every path (+ the policy's choice), oracle timed beside."""
    import numpy as np
    import torch

    from paged_kv_gqa_block_amd import engine, timing, traces

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rules = engine.load_policy_table()
    cost_model = engine.load_cost_model()
    for name in ALL_CONFIGS:
        spec = traces.get_spec(name)
        w = traces.generate(spec, traces.HELD_OUT_SEED)
        lens = w["seq_lens"].numpy()
        wd = engine.to_device(w)
        engine.validate_inputs(wd)
        views = timing.pool_copies(wd, args.copies_gib, max_copies=8)
        pol = engine.choose(rules, spec.batch, int(lens.max()))
        mod = engine.choose_model(cost_model, engine.problem_from_workload(w), lens)[:2]
        dflt = engine.choose_default(rules, cost_model, engine.problem_from_workload(w), lens)
        cands = [("bucketed", spec.splits), ("workqueue", spec.splits), ("nosplit", 1),
                 ("padded", spec.splits)]
        for c in (pol, mod, dflt):
            if c not in cands:
                cands.append(c)
        cpu = None if args.no_cpu_baseline else cpu_baseline(w, min(args.cpu_budget_s, 5.0))
        pr = timing.time_read_probe(w, views, "workqueue", spec.splits, args.steps, args.warmup)
        print(json.dumps({"workload": describe(spec, "read-only probe", spec.splits, lens),
                          "config": name, "path": "read_only_probe", "splits": spec.splits,
                          "us_per_step": round(pr["us_per_launch"], 2),
                          "GB/s": round(pr["GB/s"], 1),
                          "pct_of_peak": round(100 * pr["GB/s"] / HBM_PEAK_GBS, 1)}), flush=True)
        if spec.head_dim == 128:
            for selfplan, graph in ((False, False), (False, True), (True, False), (True, True)):
                r = timing.time_device_path(w, views, spec.splits, args.steps, args.warmup,
                                            sync_reps=5, graph=graph, selfplan=selfplan)
                kv = int(lens.astype(np.int64).sum()) * spec.num_kv_heads * spec.head_dim * 4
                gbs = kv / (r["step_us"] * 1e-6) / 1e9
                print(json.dumps({
                    "workload": describe(spec, r["path"], spec.splits, lens), "config": name,
                    "path": r["path"], "splits": spec.splits, "policy_choice": False,
                    "us_per_step": round(r["step_us"], 2), "GB/s": round(gbs, 1),
                    "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                    "split_us_per_launch": None, "launches_per_step": 2 if selfplan else 3,
                    "kv_bytes": kv,
                    "merge_state_bytes": None,
                    "sync_wall_us_incl_plan": round(r["sync_wall_us_median"], 1),
                    "cpu_oracle": None}), flush=True)
        for path, s in cands:
            r = timing.time_path(w, views, path, s, args.kernel, args.steps, args.warmup,
                                 sync_reps=5, graph=args.launch == "graph")
            kv = r["info"]["kv_bytes"]
            gbs = kv / (r["step_us"] * 1e-6) / 1e9
            print(json.dumps({
                "workload": describe(spec, path, s, lens), "config": name, "path": path,
                "splits": s, "policy_choice": (path, s) == pol, "model_choice": (path, s) == mod,
                "default_choice": (path, s) == dflt, "launch": r["launch"],
                "us_per_step": round(r["step_us"], 2), "GB/s": round(gbs, 1),
                "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                "single_step_us": r["single_step_us"],
                "split_us_per_launch": round(r["split_us"] / max(1, r["n_split_launches"]), 2),
                "launches_per_step": r["info"]["n_launches"], "kv_bytes": kv,
                "merge_state_bytes": r["info"]["merge_state_bytes"],
                "sync_wall_us_incl_plan": round(r["sync_wall_us_median"], 1),
                "cpu_oracle": None if cpu is None else {
                    "GB/s": round(cpu["value"], 3), "us_per_step": round(cpu["us_per_step_equiv"]),
                    "cores": cpu["cores"]}}), flush=True)
        del views, wd, w
        torch.cuda.empty_cache()
    return 0


def run_device(args, spec, seed, splits, w, wd, lens, selfplan=False) -> int:
    """The device-planned workqueue step (pkv_plan_device -> pkv_decode_device ->
    pkv_merge_device), or the self-planned one (pkv_decode_selfplan ->
    pkv_merge_selfplan), no host work: one JSON line of the same metric,
    without the per-kernel roofline (the launches are timed together)."""
    from paged_kv_gqa_block_amd import timing

    views = timing.pool_copies(wd, args.copies_gib)
    r = timing.time_device_path(w, views, splits, args.steps, args.warmup, repeats=1,
                                selfplan=selfplan)
    kv = int(lens.astype("int64").sum()) * spec.num_kv_heads * spec.head_dim * 2 * 2
    gbs = kv / (r["step_us"] * 1e-6) / 1e9
    print(json.dumps({
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "us_per_step": round(r["step_us"], 2),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "higher_is_better": True,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": describe(spec, ("self-planned" if selfplan else
                                               "device-planned") + " workqueue", splits, lens),
                   "seed": seed, "path": "selfplan" if selfplan else "device", "splits": splits,
                   "n_tasks": r["n_tasks"], "launches_per_step": 2 if selfplan else 3,
                   "kv_bytes": kv,
                   "sync_wall_us": round(r["sync_wall_us_median"], 1)}}), flush=True)
    return 0


# The two workloads the 70 %-of-peak target is quoted on: the long single row
# on the length-bucketed split path and the bimodal batch on the compact
# workqueue, both with up to 32 splits per row.
TARGETS = ("long", "bimodal")


def choose_path(args, spec, w, lens):
    """(path, splits) of a workload: --path / --splits, else its default."""
    from paged_kv_gqa_block_amd import engine

    path = args.path or DEFAULT_PATH.get(spec.name, "workqueue")
    splits = args.splits or spec.splits
    if path == "policy":  # the calibrated (B, N_max) table
        path, splits = engine.choose(engine.load_policy_table(), spec.batch, int(lens.max()))
    elif path == "model":  # the learned cost model's choice
        path, splits, _ = engine.choose_model(engine.load_cost_model(),
                                              engine.problem_from_workload(w), lens)
    elif path == "default":  # the engine's default policy (table for B = 1, model else)
        path, splits = engine.choose_default(engine.load_policy_table(),
                                             engine.load_cost_model(),
                                             engine.problem_from_workload(w), lens)
    return path, splits


def measure(args, w, wd, path, splits, seed, with_probe=True):
    """One workload in one launch configuration: the contract figures (K steps
    timed once) and the split kernel's roofline."""
    from paged_kv_gqa_block_amd import timing

    spec = w["spec"]
    lens = w["seq_lens"].numpy()
    kernel_used = args.kernel
    if kernel_used == "auto":  # the library's AUTO rule: matrix cores for d = 128
        kernel_used = "mfma" if spec.head_dim == 128 else "valu"
    views = timing.pool_copies(wd, args.copies_gib)
    # Exactly K steps timed once (repeats=1), launched as configured.
    r = timing.time_path(w, views, path, splits, args.kernel, args.steps, args.warmup, repeats=1,
                         graph=args.launch == "graph")
    info = r["info"]
    kv = info["kv_bytes"]
    gbs = kv / (r["step_us"] * 1e-6) / 1e9
    split_launch_us = r["split_us"] / max(1, r["n_split_launches"])
    split_gbs = (kv / max(1, r["n_split_launches"])) / (split_launch_us * 1e-6) / 1e9
    out = {
        "us_per_step": round(r["step_us"], 2), "GB/s": round(gbs, 1),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "config": {"workload": describe(spec, path, splits, lens), "seed": seed,
                   "kernel": args.kernel, "path": path, "splits": splits, "launch": r["launch"],
                   "launches_per_step": info["n_launches"], "n_tasks": info["n_tasks"],
                   "kv_bytes": kv, "merge_state_bytes": info["merge_state_bytes"],
                   "pool_copies_rotated": len(views),
                   "single_step_us": r["single_step_us"],
                   "sync_wall_us_incl_plan": round(r["sync_wall_us_median"], 1)},
        "roofline": {"bound": "hbm", "achieved": round(split_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(spec.name, kernel_used, path, splits, seed),
                     "kernel": f"split decode ({kernel_used})",
                     "launch_us": round(split_launch_us, 2),
                     "algorithmic_bytes_per_launch": kv // max(1, r["n_split_launches"])},
    }
    # The same K steps launched the other way, for comparison.
    other = timing.time_path(w, views, path, splits, args.kernel, args.steps, args.warmup,
                             repeats=1, sync_reps=0, graph=args.launch != "graph")
    out["config"][f"{other['launch']}_us_per_step"] = round(other["step_us"], 2)
    if with_probe and r["n_split_launches"] == 1:
        # The same tasks' pages streamed by a read-only kernel: the rate this
        # access pattern reaches on the device (the split kernel's ceiling).
        pr = timing.time_read_probe(w, views, path, splits, args.steps, args.warmup)
        out["roofline"]["read_only_probe"] = {
            "GB/s": round(pr["GB/s"], 1), "launch_us": round(pr["us_per_launch"], 2),
            "achieved_over_probe": round(split_gbs / pr["GB/s"], 4)}
    return out


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode path has no multi-GPU mode)", file=sys.stderr)
        return 2
    import torch

    from paged_kv_gqa_block_amd import engine, traces

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.all:
        return run_all(args)
    spec = traces.get_spec(args.config)
    seed = traces.HELD_OUT_SEED if args.seed is None else args.seed
    w = traces.generate(spec, seed)
    lens = w["seq_lens"].numpy()
    path, splits = choose_path(args, spec, w, lens)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    if path in ("device", "selfplan"):
        return run_device(args, spec, seed, splits, w, wd, lens, selfplan=path == "selfplan")

    m = measure(args, w, wd, path, splits, seed)
    line = {
        "metric": METRIC,
        "value": m["GB/s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["us_per_step"] / 1000, 5),
        "us_per_step": m["us_per_step"],
        "pct_of_peak": m["pct_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
    }
    if args.config in TARGETS and not args.no_targets:
        # Both target workloads in their default launch configuration, on the
        # same held-out seed and rotated pools.
        targets = {}
        for name in TARGETS:
            if name == args.config and args.path is None and args.splits is None:
                t = m
            else:
                del wd
                torch.cuda.empty_cache()
                tspec = traces.get_spec(name)
                w = traces.generate(tspec, seed)
                wd = engine.to_device(w)
                engine.validate_inputs(wd)
                tp = DEFAULT_PATH.get(name, "workqueue")
                t = measure(args, w, wd, tp, tspec.splits, seed)
            targets[name] = {"us_per_step": t["us_per_step"], "GB/s": t["GB/s"],
                             "pct_of_peak": t["pct_of_peak"],
                             "workload": t["config"]["workload"],
                             "launch": t["config"]["launch"],
                             "graph_us_per_step": t["config"].get("graph_us_per_step"),
                             "eager_us_per_step": t["config"].get("eager_us_per_step"),
                             "split_roofline": {k: t["roofline"][k] for k in
                                                ("achieved", "frac", "launch_us", "traffic")},
                             "read_only_probe": t["roofline"].get("read_only_probe")}
            # The engine's default policy on the same workload (its own path
            # and split cap), timed the same way.
            lens_t = w["seq_lens"].numpy()
            dpath, ds = engine.choose_default(engine.load_policy_table(),
                                              engine.load_cost_model(),
                                              engine.problem_from_workload(w), lens_t)
            tconf = (t["config"]["path"], t["config"]["splits"])
            d = t if (dpath, ds) == tconf else measure(args, w, wd, dpath, ds, seed,
                                                       with_probe=False)
            targets[name]["default_policy"] = {
                "path": dpath, "splits": ds, "us_per_step": d["us_per_step"], "GB/s": d["GB/s"],
                "pct_of_peak": d["pct_of_peak"]}
        line["targets"] = targets
        w = traces.generate(spec, seed)  # the contract workload again, for the CPU leg
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
