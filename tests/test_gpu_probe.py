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
