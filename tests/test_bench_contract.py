"""bench.py on the CPU: its command-line contract (one GPU only) and the
profile records its roofline object quotes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _bench_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_recorded_profiles_match_the_device_sources():
    """Every committed profile summary that records a source hash was taken on
    the device sources as they are now, so the counter traffic the bench line
    reports belongs to the kernel it times; and each traffic record is within
    a few per cent above the workload's algorithmic bytes."""
    import glob

    import numpy as np

    from paged_kv_gqa_block_amd import traces

    bench = _bench_module()
    want = bench.kernel_source_hash()
    hashed = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        with open(path) as f:
            text = f.read()
        assert "command" in text, path
        for line in text.splitlines():
            if line.startswith("kernel_source_sha256_16:"):
                assert line.split()[1] == want, path
                hashed += 1
    assert hashed >= len(bench.TRAFFIC_PROFILES)
    for config in bench.TRAFFIC_PROFILES:
        spec = traces.get_spec(config)
        path = bench.DEFAULT_PATH.get(config, "workqueue")
        traffic = bench.recorded_traffic(config, "mfma", path, spec.splits, traces.HELD_OUT_SEED)
        assert traffic is not None, config
        lens = traces.draw_lengths(spec, np.random.default_rng(traces.HELD_OUT_SEED))
        kv = int(lens.sum()) * spec.num_kv_heads * spec.head_dim * 2 * 2  # K and V, 2 B each
        assert 1.0 <= traffic / kv <= 1.05, (config, traffic / kv)
