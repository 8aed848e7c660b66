"""GPU: the device-planned workqueue step (pkv_plan_device, pkv_decode_device,
pkv_merge_device) against the host planner and the fp64 oracle, including
HIP-graph capture replayed with changing lengths."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_block_amd import _lib, engine, traces
from tests.parity import check_lse, check_out, oracle_out, say

pytestmark = pytest.mark.gpu
SEED = traces.HELD_OUT_SEED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _host_plan(prob, lens, s):
    buf = np.zeros(_lib.pkv_plan_bytes(prob, _lib.PKV_WORKQUEUE, s) // 4, dtype=np.int32)
    _lib.pkv_plan(prob, np.asarray(lens, np.int32), _lib.PKV_WORKQUEUE, s, buf)
    return buf


@pytest.mark.parametrize("seed", range(6))
def test_device_plan_equals_host_plan(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.choice([1, 3, 8, 64, 1500]))
    hkv = int(rng.choice([1, 2, 8]))
    s = int(rng.choice([1, 4, 32]))
    lens = rng.integers(0, 4096, size=b).astype(np.int32)
    lens[rng.random(b) < 0.15] = 0
    say(f"[device plan] seed={seed} B={b} Hkv={hkv} S={s}")
    prob = _lib.make_problem(b, hkv * 4, hkv, 128, 16, 1 << 20, 256)
    host = _host_plan(prob, lens, s)
    step = engine.DeviceStep(prob, s)
    _lib.pkv_plan_device(prob, torch.from_numpy(lens).cuda(), s, step.plan_dev,
                         bad_rows_dev=step.bad_rows)
    torch.cuda.synchronize()
    total = int(host[13])
    dev = step.plan_dev.cpu().numpy()
    assert int(dev[13]) == total
    np.testing.assert_array_equal(dev[:total], host[:total])
    assert int(step.bad_rows.item()) == 0


def test_device_plan_at_the_batch_limit():
    """16384 rows (the device planner's maximum), ~2 M tasks: word for word."""
    rng = np.random.default_rng(99)
    b, hkv, s = 16384, 8, 32
    lens = rng.integers(0, 4096, size=b, endpoint=True).astype(np.int32)
    lens[rng.random(b) < 0.1] = 0
    say(f"[device plan] B={b} Hkv={hkv} S={s}")
    prob = _lib.make_problem(b, hkv * 4, hkv, 128, 16, 1 << 20, 256)
    host = _host_plan(prob, lens, s)
    plan_dev = torch.full((host.size,), -7, dtype=torch.int32, device="cuda")  # every word used must be written
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.pkv_plan_device(prob, torch.from_numpy(lens).cuda(), s, plan_dev, bad_rows_dev=bad)
    torch.cuda.synchronize()
    total = int(host[13])
    dev = plan_dev.cpu().numpy()
    np.testing.assert_array_equal(dev[:total], host[:total])
    assert int(bad.item()) == 0
    assert int(host[6]) > 1_000_000
    assert int(dev[total]) == 0  # work counter zeroed


def _device_run(w, splits):
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.DeviceStep(engine.problem_from_workload(w), splits)
    step.run(wd)
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("name", ["long", "bimodal", "zipf", "policy_b8"])
def test_device_step_matches_oracle(name):
    w = traces.generate(traces.get_spec(name), SEED)
    say(f"[device step] {name}")
    ref_out, ref_lse = oracle_out(w)
    step = _device_run(w, w["spec"].splits)
    check_out(step.out, ref_out, w["spec"].dtype, label=name)
    check_lse(step.lse, ref_lse, label=name)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (32, 2), (4, 4)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_device_step_edge_lengths(hq, hkv, dtype):
    lens = np.array([0, 1, 15, 16, 17, 33, 100, 0, 250], dtype=np.int32)
    spec = traces.custom_spec(len(lens), hq, hkv, 128, splits=3, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[device edge] hq={hq} hkv={hkv} {dtype}")
    ref_out, ref_lse = oracle_out(w)
    for s in (3, 40):
        step = _device_run(w, s)
        check_out(step.out, ref_out, dtype, label=f"device-edge S={s}")
        check_lse(step.lse, ref_lse, label=f"device-edge S={s}")


def test_bad_lengths_are_planned_empty_and_counted():
    lens = np.array([40, 70, 33], dtype=np.int32)
    spec = traces.custom_spec(3, 8, 2, 128, splits=4)
    w = traces.generate(spec, SEED, seq_lens=lens)
    wd = engine.to_device(w)
    cap = int(w["block_table"].shape[1]) * 16  # 80 tokens
    bad = torch.tensor([40, cap + 1, -3], dtype=torch.int32, device="cuda")
    say("[device bad rows]")
    step = engine.DeviceStep(engine.problem_from_workload(w), 4)
    step.run(dict(wd, seq_lens=bad))
    torch.cuda.synchronize()
    assert int(step.bad_rows.item()) == 2
    ref_out, ref_lse = oracle_out(w, rows=[0])
    check_out(step.out, ref_out, "f16", rows=[0], label="bad-rows row 0")
    assert (step.out[1:].float() == 0).all() and torch.isneginf(step.lse[1:]).all()


def test_graph_capture_replays_with_growing_lengths():
    """Capture plan + split + merge once; replay with new device lengths."""
    final = np.array([3000, 700, 12000, 64], dtype=np.int32)
    spec = traces.custom_spec(4, 32, 8, 128, splits=16)
    w = traces.generate(spec, SEED, seq_lens=final)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.DeviceStep(engine.problem_from_workload(w), 16)
    lens_dev = torch.tensor(final // 2, dtype=torch.int32, device="cuda")
    view = dict(wd, seq_lens=lens_dev)
    say("[graph] capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run(view, stream=s)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step.run(view, stream=s)
    torch.cuda.synchronize()
    for k, frac in enumerate((0.25, 0.5, 0.75, 1.0, 0.6)):
        lens = np.maximum((final * frac).astype(np.int32), 0)
        lens_dev.copy_(torch.from_numpy(lens))
        torch.zeros(1024, device="cuda").add_(1.0)  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {k} lens={lens.tolist()}")
        w_k = dict(w, seq_lens=torch.from_numpy(lens))
        ref_out, ref_lse = oracle_out(w_k)
        check_out(step.out, ref_out, "f16", label=f"graph replay {k}")
        check_lse(step.lse, ref_lse, label=f"graph replay {k}")


def test_decode_merge_rerun_without_replanning():
    """The device merge resets the work counter, so decode + merge can run
    again on the same device plan and give the same bits."""
    w = traces.generate(traces.get_spec("bimodal"), SEED)
    wd = engine.to_device(w)
    say("[device rerun]")
    step = engine.DeviceStep(engine.problem_from_workload(w), 32)
    step.run(wd)
    torch.cuda.synchronize()
    first = step.out.clone()
    for _ in range(2):
        _lib.pkv_decode_device(step.prob, step.plan_dev, 32, wd["q"], wd["k_pool"], wd["v_pool"],
                               wd["block_table"], step.st_m, step.st_l, step.st_o)
        _lib.pkv_merge_device(step.prob, step.plan_dev, step.st_m, step.st_l, step.st_o,
                              step.out, step.lse)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), step.out.view(torch.int16))
