"""Device timing of one decode path (HIP events on the launch stream).

Used by bench.py and by the policy calibration.  A step is the engine's
device work for one decode step of one layer (split + merge launches, or the
single no-split launch) with the plan resident on the GPU.  Every step reads
the next of several copies of the KV pools, so the 256 MB Infinity Cache
cannot serve K/V from the previous step (consecutive layers of a model also
read different pools).
"""
from __future__ import annotations

import math
import statistics
import time

import numpy as np
import torch

from . import _lib, engine, probe

# Device time the host gets to enqueue a timed window before it starts: a
# sleeping wave (pkv_probe_sleep) is enqueued just before the start event,
# so the window holds the launches and not the host's first submission.
LEAD_US = 200


# MI355X's Infinity Cache (MALL) holds 256 MiB; the rotated copies always
# total at least twice that, so no step reads K/V that a recent step left there.
MALL_BYTES = 256 << 20


def pool_copies(wd: dict, copies_gib: float, max_copies: int = 64):
    """Views of the workload on n copies of the pools: n * pool size >=
    copies_gib, at most max_copies copies unless fewer would total less than
    2 x the 256 MiB Infinity Cache (small pools then get as many copies as
    that takes)."""
    pool_bytes = wd["k_pool"].numel() * wd["k_pool"].element_size() * 2
    want = math.ceil(copies_gib * (1 << 30) / pool_bytes)
    floor = math.ceil(2 * MALL_BYTES / pool_bytes)
    n = max(1, floor, min(max_copies, want))
    views = [wd]
    for _ in range(n - 1):
        views.append(dict(wd, k_pool=wd["k_pool"].clone(), v_pool=wd["v_pool"].clone()))
    return views


def _capture(fn, stream) -> torch.cuda.CUDAGraph:
    """A HIP graph of the launches fn() enqueues on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def time_path(w: dict, views, path: str, splits: int, kernel: str = "auto", steps: int = 50,
              warmup: int = 10, sync_reps: int = 20, repeats: int = 5,
              graph: bool = False) -> dict:
    """Times one (path, split cap).  Returns step / split times and counters.

    The timed loops run `repeats` times; the reported step and split times are
    the medians (short kernels vary by several percent from run to run).
    With ``graph``, the timed loop of K steps (and of K split launches) is
    captured once in a HIP graph, launched once untimed (its first launch also
    uploads it), and replayed: the same launches, enqueued by one graph launch
    instead of one host call per kernel.
    """
    wd = views[0]
    prob = engine.problem_from_workload(w, kernel)
    step = engine.DecodeStep(prob, path, splits)
    stream = torch.cuda.Stream() if graph else torch.cuda.current_stream()
    info = step.plan(wd["seq_lens_host"], stream=stream)
    n = len(views)
    torch.cuda.synchronize()
    for i in range(warmup):
        step.run(views[i % n], stream)
    torch.cuda.synchronize()

    # Arguments marshalled once per pool copy: the host then enqueues a step
    # in a few microseconds, well under the device time of the shortest steps.
    bound = [step.bind(v, stream) for v in views]

    def steps_from(base):
        for i in range(steps):
            step.run_bound(bound[(base + i) % n])

    def splits_from(base):
        for i in range(steps):
            step.decode_bound(bound[(base + i) % n])

    graphs = None
    if graph:
        # Captured once; the first launch of a graph also uploads it to the
        # device, so each is launched once untimed before the timed replays.
        graphs = (_capture(lambda: steps_from(warmup), stream),
                  _capture(lambda: splits_from(warmup + steps), stream))
        with torch.cuda.stream(stream):  # replays run on the capture stream
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
    step_runs, split_runs = [], []
    for rep in range(repeats):
        base = warmup + rep * 2 * steps
        if graphs is not None:
            run_steps, run_splits = graphs[0].replay, graphs[1].replay
        else:
            run_steps = lambda: steps_from(base)  # noqa: E731
            run_splits = lambda: splits_from(base + steps)  # noqa: E731
        # K back-to-back steps between two events (no event between launches).
        with torch.cuda.stream(stream):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            probe.probe_sleep(LEAD_US, stream)
            e0.record(stream)
            run_steps()
            e1.record(stream)
            torch.cuda.synchronize()
            step_runs.append(1e3 * e0.elapsed_time(e1) / steps)

            # Split launches alone, back to back, so event overhead is amortised.
            e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            probe.probe_sleep(LEAD_US, stream)
            e2.record(stream)
            run_splits()
            e3.record(stream)
            torch.cuda.synchronize()
            split_runs.append(1e3 * e2.elapsed_time(e3) / steps)
    step_us = statistics.median(step_runs)
    split_us = statistics.median(split_runs)

    # Distribution of single steps: an event pair around each step of one
    # more loop (the events add a little time to each step, so the
    # throughput figures above come from the back-to-back loops).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            step.run(views[(warmup + i) % n], stream)
            b.record(stream)
    torch.cuda.synchronize()
    single = sorted(1e3 * a.elapsed_time(b) for a, b in evs)

    def pct(q):
        return single[min(len(single) - 1, int(round(q * (len(single) - 1))))]

    # Synchronised wall time per step including host planning and the plan
    # upload (the pages' end-to-end latency metric).
    sync_us = []
    for i in range(sync_reps):
        torch.cuda.synchronize()
        t = time.perf_counter()
        step.plan(wd["seq_lens_host"], stream=stream)
        step.run(views[i % n], stream)
        torch.cuda.synchronize()
        sync_us.append((time.perf_counter() - t) * 1e6)

    n_split = {0: info.n_buckets, 1: 1 if info.n_tasks else 0, 2: 1, 3: info.n_buckets}[info.path]
    return {
        "path": path,
        "splits": splits,
        "info": info.as_dict(),
        "n_split_launches": n_split,
        "step_us": step_us,
        "split_us": split_us,
        "step_us_runs": [round(x, 2) for x in step_runs],
        "launch": "graph" if graph else "eager",
        "single_step_us": {"p10": round(pct(0.1), 2), "p50": round(pct(0.5), 2),
                           "p90": round(pct(0.9), 2), "n": len(single)},
        "sync_wall_us_median": statistics.median(sync_us) if sync_us else None,
        "out": step.out,
    }


def time_paths_interleaved(w: dict, views, configs, kernel: str = "auto", steps: int = 30,
                           warmup: int = 5, repeats: int = 7, return_runs: bool = False):
    """Step time of several (path, split cap) configurations of one workload.

    Each configuration's K steps (rotating over the pool copies) are captured
    once in a HIP graph and replayed per timed repeat, so the host, whose
    eager launches cost a few microseconds each, never holds the device back
    on short steps.  The timed repeats alternate between the configurations
    (repeat r of every configuration before repeat r + 1 of any), so a drift
    of the GPU's clock moves all of them alike; each result is the median
    over its repeats.  Returns {"path:splits": step_us}, and with
    ``return_runs`` also {"path:splits": [µs of each repeat]} and the host
    time to launch one replay, per step.
    """
    prob = engine.problem_from_workload(w, kernel)
    stream = torch.cuda.Stream()
    n = len(views)
    steps_by = {}
    for path, s in configs:
        st = engine.DecodeStep(prob, path, s)
        st.plan(views[0]["seq_lens_host"], stream=stream)
        bound = [st.bind(v, stream) for v in views]  # arguments marshalled once
        for i in range(warmup):
            st.run_bound(bound[i % n])
        torch.cuda.synchronize()
        graph = _capture(lambda st=st, bound=bound: [st.run_bound(bound[i % n])
                                                       for i in range(steps)], stream)
        with torch.cuda.stream(stream):
            graph.replay()  # the first launch also uploads the graph: untimed
        torch.cuda.synchronize()
        steps_by[f"{path}:{s}"] = (st, graph)
    torch.cuda.synchronize()
    runs = {k: [] for k in steps_by}
    host = {k: [] for k in steps_by}
    with torch.cuda.stream(stream):
        for _rep in range(repeats):
            for key, (_st, graph) in steps_by.items():
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                probe.probe_sleep(LEAD_US, stream)
                e0.record(stream)
                t0 = time.perf_counter()
                graph.replay()
                host[key].append((time.perf_counter() - t0) * 1e6 / steps)
                e1.record(stream)
                torch.cuda.synchronize()
                runs[key].append(1e3 * e0.elapsed_time(e1) / steps)
    med = {k: statistics.median(v) for k, v in runs.items()}
    if return_runs:
        return med, runs, {k: statistics.median(v) for k, v in host.items()}
    return med


def time_read_probe(w: dict, views, path: str, splits: int, steps: int = 50,
                    warmup: int = 10, repeats: int = 5) -> dict:
    """Read-only probe over the pages of one plan's tasks (libpkv_probe.so):
    the HBM rate of the split kernel's access pattern with no compute.
    Returns the median µs per probe launch and the real-KV GB/s it implies."""
    prob = engine.problem_from_workload(w, "auto")
    step = engine.DecodeStep(prob, path, splits)
    stream = torch.cuda.current_stream()
    info = step.plan(views[0]["seq_lens_host"], stream=stream)
    sink = torch.zeros(max(1, info.n_tasks), dtype=torch.int32, device="cuda")
    n = len(views)
    for i in range(warmup):
        probe.probe_read(views[i % n], step, sink, stream)
    torch.cuda.synchronize()
    runs = []
    for rep in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe.probe_sleep(LEAD_US, stream)
        e0.record(stream)
        for i in range(steps):
            probe.probe_read(views[(warmup + rep * steps + i) % n], step, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        runs.append(1e3 * e0.elapsed_time(e1) / steps)
    us = statistics.median(runs)
    return {"us_per_launch": us, "GB/s": info.kv_bytes / (us * 1e-6) / 1e9,
            "n_tasks": info.n_tasks}


def time_device_path(w: dict, views, splits: int, steps: int = 50, warmup: int = 10,
                     sync_reps: int = 20, repeats: int = 5, graph: bool = False,
                     selfplan: bool = False) -> dict:
    """Times the device-planned workqueue step (plan + persistent split + merge
    on the GPU, no host work), or with ``selfplan`` the self-planned step
    (persistent split + merge deriving the workqueue in-kernel).  With
    ``graph``, each pool copy's step is captured once in a HIP graph and
    replayed."""
    prob = engine.problem_from_workload(w, "auto")
    step = (engine.SelfPlannedStep if selfplan else engine.DeviceStep)(prob, splits)
    n = len(views)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step.run(views[i % n], stream)
    torch.cuda.synchronize()
    graphs = None
    if graph:
        graphs = []
        for v in views:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step.run(v, stream)
            graphs.append(g)
        with torch.cuda.stream(stream):  # the first launch also uploads a graph: untimed
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()

    def one(i):
        if graphs is None:
            step.run(views[i % n], stream)
        else:
            graphs[i % n].replay()

    runs = []
    with torch.cuda.stream(stream):
        for rep in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            probe.probe_sleep(LEAD_US, stream)
            e0.record(stream)
            for i in range(steps):
                one(warmup + rep * steps + i)
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(1e3 * e0.elapsed_time(e1) / steps)
        sync_us = []
        for i in range(sync_reps):
            torch.cuda.synchronize()
            t = time.perf_counter()
            one(i)
            torch.cuda.synchronize()
            sync_us.append((time.perf_counter() - t) * 1e6)
    # Task count of the same workqueue, from the library's host planner (host
    # plan only, no device copy).
    lens = np.ascontiguousarray(w["seq_lens"].numpy(), dtype=np.int32)
    plan_host = np.zeros(_lib.pkv_plan_bytes(prob, _lib.PKV_WORKQUEUE, splits) // 4, np.int32)
    n_tasks = int(_lib.pkv_plan(prob, lens, _lib.PKV_WORKQUEUE, splits, plan_host).n_tasks)
    return {
        "path": ("workqueue_selfplan" if selfplan else "workqueue_device") +
                ("_graph" if graph else ""),
        "splits": splits,
        "n_tasks": n_tasks,
        "step_us": statistics.median(runs),
        "step_us_runs": [round(x, 2) for x in runs],
        "sync_wall_us_median": statistics.median(sync_us) if sync_us else None,
        "out": step.out,
    }
