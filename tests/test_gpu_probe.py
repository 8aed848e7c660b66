"""The read-only bandwidth probe (libpkv_probe.so) runs on a plan's tasks."""
import pytest
import torch

from paged_kv_gqa_block_amd import engine, traces
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,path", [("tiny", "workqueue"), ("bimodal", "bucketed")])
def test_probe_reads_plan_pages(name, path):
    from paged_kv_gqa_block_amd import probe

    w = traces.generate(traces.get_spec(name), traces.HELD_OUT_SEED)
    say(f"[probe] {name} {path}")
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.DecodeStep(engine.problem_from_workload(w, "auto"), path, w["spec"].splits)
    info = step.plan(wd["seq_lens_host"])
    sink = torch.zeros(info.n_tasks, dtype=torch.int32, device="cuda")
    probe.probe_read(wd, step, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def _lds_probe_expected(w, tasks, waves):
    """Per (task, wave, lane) checksum of the pages pkv_probe_read_lds moves
    (numpy, from the host copies of the pools): bytes past a page's last real
    token count as zero, as the probe's buffer bounds return them."""
    import numpy as np

    def chunk_xor(pool):
        a = pool.contiguous().view(torch.int32).numpy().view(np.uint32)
        a = a.reshape(a.shape[0], a.shape[1], 4, 64, 4)  # [page][head][chunk i][lane][word]
        return (a[..., 0] ^ a[..., 1] ^ a[..., 2] ^ a[..., 3]).astype(np.uint64)

    c = chunk_xor(w["k_pool"]) + chunk_xor(w["v_pool"])
    token = (np.arange(4)[:, None] * 4 + np.arange(64)[None, :] // 16)  # token of chunk (i, lane)
    bt = w["block_table"].numpy()
    out = np.zeros((len(tasks), waves, 64), dtype=np.uint64)
    for t, (row, gs, pb, te) in enumerate(tasks):
        g, pe = gs >> 16, (te + 15) // 16
        for wv in range(waves):
            for idx in range(pb + wv, pe, waves):
                valid = min(16, te - idx * 16)
                out[t, wv] += (c[bt[row, idx], g] * (token < valid)).sum(axis=0)
    return (out & 0xFFFFFFFF).astype(np.uint32)


@pytest.mark.parametrize("name,path", [("bimodal", "workqueue"), ("zipf", "bucketed")])
def test_lds_ring_probe_reads_plan_pages(name, path):
    """The direct-to-LDS probe moves exactly the plan's pages: its per-lane
    checksums equal the ones computed on the host, for every ring shape."""
    import numpy as np

    from paged_kv_gqa_block_amd import probe

    w = traces.generate(traces.get_spec(name), traces.HELD_OUT_SEED)
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.DecodeStep(engine.problem_from_workload(w, "auto"), path, w["spec"].splits)
    info = step.plan(wd["seq_lens_host"])
    ph = step.plan_host.numpy()
    tasks = ph[ph[10]:ph[10] + 4 * info.n_tasks].reshape(-1, 4)
    for waves, depth in probe.LDS_SHAPES:
        say(f"[probe lds] {name} {path} waves={waves} depth={depth}")
        sink = torch.zeros(info.n_tasks * waves * 64, dtype=torch.int32, device="cuda")
        probe.probe_read_lds(wd, step, waves, depth, True, sink)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32).reshape(-1, waves, 64)
        assert (got == _lds_probe_expected(w, tasks, waves)).all()
        probe.probe_read_lds(wd, step, waves, depth, False, sink)
        torch.cuda.synchronize()
        assert int(sink.abs().sum()) == 0


def test_stream_and_empty_probes():
    from paged_kv_gqa_block_amd import probe

    say("[probe] stream + empty")
    buf = torch.randn(1 << 22, device="cuda")  # 16 MiB
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    for grid, u in ((256, 4), (512, 8)):
        probe.probe_stream(buf, 1 << 24, grid, u, sink)
    with pytest.raises(RuntimeError):
        probe.probe_stream(buf, 1000, 256, 4, sink)  # not a multiple of the grid's loads
    flag = torch.tensor([7, 0], dtype=torch.int32, device="cuda")
    probe.probe_empty(32, 256, flag)
    torch.cuda.synchronize()
    assert flag.tolist() == [7, 7] and int(sink.abs().sum()) == 0


def test_sleep_probe_holds_the_device():
    """pkv_probe_sleep keeps the stream busy for about the requested time and
    then ends; out-of-range durations are rejected on the host."""
    from paged_kv_gqa_block_amd import probe

    say("[probe] sleep")
    s = torch.cuda.current_stream()
    for us in (0, 100, 400):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        probe.probe_sleep(us, s)
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        assert 0.8 * us / 1e3 <= ms < us / 1e3 + 5.0, (us, ms)
    with pytest.raises(RuntimeError):
        probe.probe_sleep(-1)
    with pytest.raises(RuntimeError):
        probe.probe_sleep(60000)
