"""GPU: KV append through the block table (pkv_append_kv), alone and in a
multi-step decode loop, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_block_amd import _lib, engine, traces
from tests.parity import check_lse, check_out, oracle_out, say

pytestmark = pytest.mark.gpu
SEED = traces.HELD_OUT_SEED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d,dtype", [(128, "f16"), (64, "bf16")])
def test_append_matches_oracle_bit_exactly(d, dtype):
    lens = np.array([33, 16, 0, 200], dtype=np.int32)
    spec = traces.custom_spec(4, 8, 2, d, splits=4, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=lens)
    wd = engine.to_device(w)
    cap = int(w["block_table"].shape[1]) * 16
    positions = np.array([32, 15, -1, cap], dtype=np.int32)  # inactive row, past capacity
    rng = np.random.default_rng(5)
    k_new = torch.from_numpy(rng.standard_normal((4, 2, d), dtype=np.float32)).to(
        wd["q"].dtype).cuda()
    v_new = torch.from_numpy(rng.standard_normal((4, 2, d), dtype=np.float32)).to(
        wd["q"].dtype).cuda()
    say(f"[append] d={d} {dtype}")
    prob = engine.problem_from_workload(w)
    _lib.pkv_append_kv(prob, k_new, v_new, wd["block_table"],
                       torch.from_numpy(positions).cuda(), wd["k_pool"], wd["v_pool"])
    torch.cuda.synchronize()
    ok_pos = np.where(positions >= cap, -1, positions)
    ref_k, ref_v = oracle.append_kv(_bits(w["k_pool"]), _bits(w["v_pool"]),
                                    w["block_table"].numpy(), ok_pos, _bits(k_new.cpu()),
                                    _bits(v_new.cpu()), 16)
    np.testing.assert_array_equal(_bits(wd["k_pool"]), ref_k)
    np.testing.assert_array_equal(_bits(wd["v_pool"]), ref_v)


def test_decode_loop_append_then_attend():
    """Four decode steps: append each row's new K/V at its length, grow the
    lengths, attend through the policy's path; every step against the oracle."""
    start = np.array([15, 100, 0, 4096], dtype=np.int32)
    steps = 4
    spec = traces.custom_spec(4, 32, 8, 128, splits=32)
    w = traces.generate(spec, SEED, seq_lens=start + steps)  # table covers the growth
    wd = engine.to_device(w)
    prob = engine.problem_from_workload(w)
    rules = engine.load_policy_table()
    rng = np.random.default_rng(9)
    k_host, v_host = _bits(w["k_pool"]), _bits(w["v_pool"])
    lens = start.copy()
    for t in range(steps):
        k_new = torch.from_numpy(rng.standard_normal((4, 8, 128), dtype=np.float32)).half()
        v_new = torch.from_numpy(rng.standard_normal((4, 8, 128), dtype=np.float32)).half()
        pos = torch.from_numpy(lens.copy())
        _lib.pkv_append_kv(prob, k_new.cuda(), v_new.cuda(), wd["block_table"], pos.cuda(),
                           wd["k_pool"], wd["v_pool"])
        k_host, v_host = oracle.append_kv(k_host, v_host, w["block_table"].numpy(), lens,
                                          _bits(k_new), _bits(v_new), 16)
        lens = lens + 1
        path, s = engine.choose(rules, 4, int(lens.max()))
        say(f"[decode loop] step {t} lens={lens.tolist()} path={path}:{s}")
        step = engine.DecodeStep(prob, path, s)
        wd["seq_lens"] = torch.from_numpy(lens).cuda()
        step.plan(lens)
        step.run(wd)
        torch.cuda.synchronize()
        w_ref = dict(w, seq_lens=torch.from_numpy(lens),
                     k_pool=torch.from_numpy(k_host.view(np.int16)).view(torch.float16),
                     v_pool=torch.from_numpy(v_host.view(np.int16)).view(torch.float16))
        ref_out, ref_lse = oracle_out(w_ref)
        check_out(step.out, ref_out, "f16", label=f"loop step {t}")
        check_lse(step.lse, ref_lse, label=f"loop step {t}")
