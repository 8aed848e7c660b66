"""Where a decode step's time goes: read ceilings and launch floors.

    python -m paged_kv_gqa_block_amd.ceiling [--config long] [--path bucketed] [--splits 32]
                                             [--steps 40] [--repeats 7]

On one workload in one launch configuration, times loops of K launches, each
captured once in a HIP graph and replayed (device time; the K launches rotate
over copies of the KV pools larger than the Infinity Cache), with the timed
repeats of all loops interleaved:

* ``step``: the engine's step, split kernel + merge (pkv_decode + pkv_merge);
* ``split``: the split kernel alone;
* ``split+empty``: the split kernel followed by a kernel of the merge's grid
  that does nothing (pkv_probe_empty), i.e. the cost of a dependent launch
  without the merge's work;
* ``empty``: that kernel alone, and a one-workgroup kernel that copies one
  word (the cheapest dependent kernel);
* ``probe``: the read-only probe over the same tasks' pages, registers as
  staging (pkv_probe_read, the bench's probe);
* ``lds``: the same pages moved by direct-to-LDS loads into rings of 2-7
  pages per wave (pkv_probe_read_lds), with and without reading them back;
* ``stream``: a contiguous read of the same byte count with no block table
  (pkv_probe_stream), over several grids: the rate HBM gives a plain
  sequential reader of that size.

One JSON line per loop (µs per launch or step, GB/s of the workload's real
KV bytes), then a text summary.  A measurement tool; the decode path does not
use it.
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys

import torch

from . import engine, probe, timing, traces


def _loops(w, views, step, bound, stream, kv_bytes, hq_rows):
    """name -> function enqueuing one launch (or step) number i."""
    n = len(views)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    flag = torch.zeros(2, dtype=torch.int32, device="cuda")
    copies = 5
    buf = torch.empty(copies * kv_bytes, dtype=torch.uint8, device="cuda")
    loops = {
        "step (split + merge)": lambda i: step.run_bound(bound[i % n]),
        "split kernel alone": lambda i: step.decode_bound(bound[i % n]),
        "split + empty kernel of the merge's grid": lambda i: (
            step.decode_bound(bound[i % n]), probe.probe_empty(hq_rows, 256, None, stream)),
        "empty kernel of the merge's grid": lambda i: probe.probe_empty(hq_rows, 256, None,
                                                                         stream),
        "one-workgroup kernel (one load, one store)": lambda i: probe.probe_empty(1, 64, flag,
                                                                                  stream),
        "read probe, register ring (4 waves, 2 pages each)": lambda i: probe.probe_read(
            views[i % n], step, sink, stream),
    }
    for waves, depth in probe.LDS_SHAPES:
        for consume in (False, True):
            name = (f"read probe, LDS ring ({waves} waves, {depth} pages each, "
                    f"{waves * depth * 8} KiB{', read back' if consume else ''})")
            loops[name] = (lambda i, wv=waves, d=depth, c=consume: probe.probe_read_lds(
                views[i % n], step, wv, d, c, sink, stream))
    nbytes = {}
    for grid in (256, 512, 1024, 2048):
        for u in (4, 8):
            # The largest byte count within the workload's that the grid splits evenly.
            nb = kv_bytes - kv_bytes % (grid * 4096 * u)
            name = f"contiguous read of the same bytes (grid {grid}, {u} loads in flight)"
            nbytes[name] = nb
            loops[name] = (lambda i, g=grid, uu=u, nb=nb: probe.probe_stream(
                buf[(i % copies) * kv_bytes:], nb, g, uu, sink, stream))
    return loops, nbytes, (sink, flag, buf)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--config", default="long")
    ap.add_argument("--path", default="bucketed")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=7)
    args = ap.parse_args(argv)
    assert torch.cuda.is_available(), "ceiling needs a GPU"
    spec = traces.get_spec(args.config)
    if spec.head_dim != 128:
        raise SystemExit("the LDS-ring probe covers head_dim 128 only")
    w = traces.generate(spec, traces.HELD_OUT_SEED)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    views = timing.pool_copies(wd, 1.0)
    stream = torch.cuda.Stream()
    step = engine.DecodeStep(engine.problem_from_workload(w), args.path,
                             args.splits or spec.splits)
    info = step.plan(wd["seq_lens_host"], stream=stream)
    if info.n_buckets > 1 and info.path != engine.PATH_IDS["workqueue"]:
        raise SystemExit("one split launch per step expected (a single bucket or the workqueue)")
    kv = int(info.kv_bytes)
    bound = [step.bind(v, stream) for v in views]
    loops, nbytes, keep = _loops(w, views, step, bound, stream, kv,
                                 spec.batch * spec.num_q_heads)
    graphs = {}
    for name, f in loops.items():
        for i in range(args.warmup):
            with torch.cuda.stream(stream):
                f(i)
        torch.cuda.synchronize()
        g = timing._capture(lambda f=f: [f(args.warmup + i) for i in range(args.steps)], stream)
        with torch.cuda.stream(stream):
            g.replay()  # the first launch also uploads the graph: untimed
        torch.cuda.synchronize()
        graphs[name] = g
    runs = {k: [] for k in graphs}
    with torch.cuda.stream(stream):
        for _ in range(args.repeats):
            for name, g in graphs.items():
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                probe.probe_sleep(timing.LEAD_US, stream)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                runs[name].append(1e3 * e0.elapsed_time(e1) / args.steps)
    med = {k: statistics.median(v) for k, v in runs.items()}
    reads = [k for k in med if k.startswith(("read probe", "contiguous"))]
    for name, us in med.items():
        moved = nbytes.get(name, kv)  # bytes a loop iteration reads
        print(json.dumps({"config": args.config, "path": args.path,
                          "splits": args.splits or spec.splits, "loop": name,
                          "us": round(us, 2), "bytes": moved if name in reads else None,
                          "GB/s": round(moved / us / 1e3, 1) if (name in reads or "split" in name
                                                                  or "step" in name) else None,
                          "runs_us": [round(x, 2) for x in runs[name]]}), flush=True)
    step_us = med["step (split + merge)"]
    split_us = med["split kernel alone"]
    empty_after = med["split + empty kernel of the merge's grid"]
    best_lds = min((k for k in reads if "LDS" in k), key=med.get)
    best_stream = min((k for k in reads if k.startswith("contiguous")),
                      key=lambda k: med[k] / nbytes[k])
    print(f"# {args.config} ({args.path}, S={args.splits or spec.splits}): "
          f"{kv} bytes of real KV per step", flush=True)
    print(f"# step {step_us:.2f} us = split {split_us:.2f} + merge {step_us - split_us:.2f} "
          f"(dependent launch {empty_after - split_us:.2f}, merge work "
          f"{step_us - empty_after:.2f})", flush=True)
    print(f"# read ceilings: register-ring probe {med[reads[0]]:.2f} us, best LDS ring "
          f"{med[best_lds]:.2f} us ({best_lds}), best contiguous read "
          f"{med[best_stream] * kv / nbytes[best_stream]:.2f} us for the same bytes "
          f"({best_stream})", flush=True)
    del keep
    return 0


if __name__ == "__main__":
    sys.exit(main())
