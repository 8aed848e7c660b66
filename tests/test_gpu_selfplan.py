"""GPU: the self-planned workqueue step (pkv_decode_selfplan, pkv_merge_selfplan)
against the fp64 oracle and, bit for bit, against the device-planned step,
whose tasks and slots it derives in-kernel."""
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


def _run(cls, w, splits, wd=None):
    wd = wd or engine.to_device(w)
    engine.validate_inputs(wd)
    step = cls(engine.problem_from_workload(w), splits)
    step.run(wd)
    torch.cuda.synchronize()
    return step, wd


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


@pytest.mark.parametrize("name", ["long", "bimodal", "zipf", "policy_b8"])
def test_selfplan_step_matches_oracle(name):
    w = traces.generate(traces.get_spec(name), SEED)
    say(f"[selfplan] {name}")
    ref_out, ref_lse = oracle_out(w)
    step, _ = _run(engine.SelfPlannedStep, w, w["spec"].splits)
    check_out(step.out, ref_out, w["spec"].dtype, label=name)
    check_lse(step.lse, ref_lse, label=name)
    assert int(step.counter.item()) == 0  # the merge reset the claim counter


@pytest.mark.parametrize("seed", range(8))
def test_selfplan_is_bit_identical_to_the_device_planned_step(seed):
    """Same tasks, same slots, same kernel body: states and outputs agree bit
    for bit with pkv_plan_device + pkv_decode_device + pkv_merge_device."""
    rng = np.random.default_rng(500 + seed)
    b = int(rng.choice([1, 2, 5, 64, 300, 1024]))
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8, 16]))
    s = int(rng.choice([1, 3, 16, 32, 64]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hi = 3000 if b <= 64 else 400
    lens = rng.integers(0, hi, size=b).astype(np.int32)
    lens[rng.random(b) < 0.1] = 0
    spec = traces.custom_spec(b, hkv * g, hkv, 128, splits=s, dtype=dtype)
    w = traces.generate(spec, SEED + seed, seq_lens=lens)
    say(f"[selfplan == device] seed={seed} B={b} Hkv={hkv} G={g} S={s} {dtype}")
    dev, wd = _run(engine.DeviceStep, w, s)
    n_tasks = int(dev.plan_dev[6].item())
    sp, _ = _run(engine.SelfPlannedStep, w, s, wd)
    for name in ("st_m", "st_l", "st_o"):
        assert _same_bits(getattr(sp, name)[:n_tasks], getattr(dev, name)[:n_tasks]), name
    assert _same_bits(sp.out, dev.out) and _same_bits(sp.lse, dev.lse)
    rows = sorted({0, b - 1, int(lens.argmax())})
    ref_out, ref_lse = oracle_out(w, rows=rows)
    check_out(sp.out, ref_out, dtype, rows=rows, label=f"selfplan seed {seed}")
    check_lse(sp.lse, ref_lse, rows=rows, label=f"selfplan seed {seed}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (32, 2), (4, 4)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_selfplan_edge_lengths(hq, hkv, dtype):
    lens = np.array([0, 1, 15, 16, 17, 33, 100, 0, 250], dtype=np.int32)
    spec = traces.custom_spec(len(lens), hq, hkv, 128, splits=3, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[selfplan edge] hq={hq} hkv={hkv} {dtype}")
    ref_out, ref_lse = oracle_out(w)
    wd = engine.to_device(w)
    for s in (3, 40):
        step, _ = _run(engine.SelfPlannedStep, w, s, wd)
        check_out(step.out, ref_out, dtype, label=f"selfplan-edge S={s}")
        check_lse(step.lse, ref_lse, label=f"selfplan-edge S={s}")


def test_selfplan_bad_lengths_are_empty_rows():
    lens = np.array([40, 70, 33], dtype=np.int32)
    spec = traces.custom_spec(3, 8, 2, 128, splits=4)
    w = traces.generate(spec, SEED, seq_lens=lens)
    wd = engine.to_device(w)
    cap = int(w["block_table"].shape[1]) * 16  # 80 tokens
    bad = torch.tensor([40, cap + 1, -3], dtype=torch.int32, device="cuda")
    say("[selfplan bad rows]")
    step = engine.SelfPlannedStep(engine.problem_from_workload(w), 4)
    step.run(dict(wd, seq_lens=bad))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_out(w, rows=[0])
    check_out(step.out, ref_out, "f16", rows=[0], label="selfplan bad-rows row 0")
    assert (step.out[1:].float() == 0).all() and torch.isneginf(step.lse[1:]).all()


def test_selfplan_all_rows_empty():
    lens = np.zeros(5, dtype=np.int32)
    spec = traces.custom_spec(5, 32, 8, 128, splits=8)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say("[selfplan empty]")
    step, _ = _run(engine.SelfPlannedStep, w, 8)
    assert (step.out.float() == 0).all() and torch.isneginf(step.lse).all()


def test_selfplan_reruns_give_the_same_bits():
    """The merge resets the claim counter, so the step can run again (here
    with more tasks than the persistent grid, so tasks are claimed)."""
    w = traces.generate(traces.get_spec("policy_b16"), SEED)
    say("[selfplan rerun]")
    step, wd = _run(engine.SelfPlannedStep, w, 32)
    assert 16 * 8 * 32 > 3 * 256  # the grid does not cover every task
    first = step.out.clone()
    for _ in range(2):
        step.run(wd)
        torch.cuda.synchronize()
        assert _same_bits(first, step.out)
        assert int(step.counter.item()) == 0


def test_selfplan_graph_capture_replays_with_growing_lengths():
    """Capture split + merge once; replay with new device lengths (no host
    work, no memset in the graph)."""
    final = np.array([3000, 700, 12000, 64], dtype=np.int32)
    spec = traces.custom_spec(4, 32, 8, 128, splits=16)
    w = traces.generate(spec, SEED, seq_lens=final)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.SelfPlannedStep(engine.problem_from_workload(w), 16)
    lens_dev = torch.tensor(final // 2, dtype=torch.int32, device="cuda")
    view = dict(wd, seq_lens=lens_dev)
    say("[selfplan graph] capture")
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
        say(f"[selfplan graph] replay {k} lens={lens.tolist()}")
        w_k = dict(w, seq_lens=torch.from_numpy(lens))
        ref_out, ref_lse = oracle_out(w_k)
        check_out(step.out, ref_out, "f16", label=f"selfplan graph replay {k}")
        check_lse(step.lse, ref_lse, label=f"selfplan graph replay {k}")


@pytest.mark.parametrize("d,kernel,hq,hkv", [(64, "auto", 8, 2), (64, "auto", 64, 8),
                                              (128, "valu", 32, 8), (128, "valu", 16, 16)])
def test_device_steps_on_the_vector_alu_kernel(d, kernel, hq, hkv):
    """Both device-side steps (planned and self-planned) on the vector-ALU
    kernel (d = 64, or asked for explicitly): against the oracle and bit for
    bit against each other, with more tasks than the persistent grid."""
    rng = np.random.default_rng(d + hq)
    lens = rng.integers(0, 6000, size=24).astype(np.int32)
    lens[::7] = 0
    spec = traces.custom_spec(24, hq, hkv, d, splits=32, dtype="bf16" if hq == 64 else "f16")
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[valu device steps] d={d} {kernel} hq={hq} hkv={hkv}")
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    prob = engine.problem_from_workload(w, kernel)
    steps = []
    for cls in (engine.DeviceStep, engine.SelfPlannedStep):
        st = cls(prob, 32)
        st.run(wd)
        torch.cuda.synchronize()
        steps.append(st)
    assert _same_bits(steps[0].out, steps[1].out) and _same_bits(steps[0].lse, steps[1].lse)
    rows = sorted({0, 1, int(lens.argmax()), 23})
    ref_out, ref_lse = oracle_out(w, rows=rows)
    for st in steps:
        check_out(st.out, ref_out, spec.dtype, rows=rows, label=f"valu {type(st).__name__}")
        check_lse(st.lse, ref_lse, rows=rows, label=f"valu {type(st).__name__}")


@pytest.mark.parametrize("seed", range(6))
def test_selfplan_equal_split_counts(seed):
    """Every row with the same split count and B * Hkv a multiple of 8 (most
    draws): the self-planned grid starts each workgroup on a task of the
    XCD-affine order.  States and outputs equal the host-planned workqueue's
    bit for bit (same tasks, same slots, same task body), and the output
    matches the oracle."""
    rng = np.random.default_rng(8200 + seed)
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 4, 8]))
    b = int(rng.choice([1, 2, 4, 8, 12]))
    s = int(rng.choice([4, 16, 32]))
    dtype = str(rng.choice(["f16", "bf16"]))
    tmax = int(rng.integers(2, 300))
    pps = max(1, -(-tmax // s))
    ns = -(-tmax // pps)
    pages = rng.integers((ns - 1) * pps + 1, tmax + 1, size=b)
    pages[0] = tmax
    lens = ((pages - 1) * 16 + rng.integers(1, 17, size=b)).astype(np.int32)
    spec = traces.custom_spec(b, hkv * g, hkv, 128, splits=s, dtype=dtype)
    w = traces.generate(spec, SEED + seed, seq_lens=lens)
    say(f"[selfplan equal splits] seed={seed} B={b} Hkv={hkv} G={g} S={s} ns={ns} {dtype}")
    sp, wd = _run(engine.SelfPlannedStep, w, s)
    host = engine.DecodeStep(engine.problem_from_workload(w), "workqueue", s)
    info = host.plan(wd["seq_lens_host"])
    host.run(wd)
    torch.cuda.synchronize()
    n_tasks = int(info.n_tasks)
    assert n_tasks == b * hkv * ns
    for name in ("st_m", "st_l", "st_o"):
        assert _same_bits(getattr(sp, name)[:n_tasks], getattr(host, name)[:n_tasks]), name
    assert _same_bits(sp.out, host.out) and _same_bits(sp.lse, host.lse)
    ref_out, ref_lse = oracle_out(w)
    check_out(sp.out, ref_out, dtype, label=f"selfplan-equal {seed}")
    check_lse(sp.lse, ref_lse, label=f"selfplan-equal {seed}")
