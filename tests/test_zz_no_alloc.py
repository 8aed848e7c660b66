"""GPU: pkv_attend_noalloc, the self-planned step with its partial states in
the library's own device array (no allocation), through the C ABI against the
existing entry points it varies (pkv_decode_selfplan + pkv_merge_selfplan)
and against the fp64 oracle: two calls in a row, the second one smaller, so
the second reads nothing the first left in the array."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_block_amd import _lib, engine, traces
from tests.parity import check_lse, check_out, oracle_out, say

pytestmark = pytest.mark.gpu
SEED = traces.HELD_OUT_SEED


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


def _noalloc(w, wd, splits):
    prob = engine.problem_from_workload(w)
    spec = w["spec"]
    dt = engine.TORCH_DTYPE[spec.dtype]
    out = torch.full((spec.batch, spec.num_q_heads, spec.head_dim), float("nan"), dtype=dt,
                     device="cuda")
    lse = torch.full((spec.batch, spec.num_q_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    assert 0 < _lib.pkv_noalloc_bytes(prob, splits) <= _lib.PKV_NOALLOC_SCRATCH_BYTES
    _lib.pkv_attend_noalloc(prob, wd["seq_lens"], splits, wd["q"], wd["k_pool"], wd["v_pool"],
                            wd["block_table"], out, lse)
    return out, lse


CALLS = [
    # (batch, Hq, Hkv, d, dtype, split cap, lengths); the second call is smaller
    (8, 32, 8, 128, "f16", 32, [1500, 20000, 130, 32768, 700, 16400, 2048, 30000]),
    (3, 16, 4, 128, "bf16", 8, [600, 0, 1001]),
]


def test_noalloc_matches_selfplanned_step_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    for b, hq, hkv, d, dtype, s, lens in CALLS:
        lens = np.asarray(lens, dtype=np.int32)
        spec = traces.custom_spec(b, hq, hkv, d, splits=s, dtype=dtype)
        w = traces.generate(spec, SEED, seq_lens=lens)
        say(f"[noalloc] B={b} Hq={hq} Hkv={hkv} d={d} {dtype} S={s} lens={lens.tolist()}")
        wd = engine.to_device(w)
        engine.validate_inputs(wd)
        out, lse = _noalloc(w, wd, s)
        ref = engine.SelfPlannedStep(engine.problem_from_workload(w), s)
        ref.run(wd)
        torch.cuda.synchronize()
        assert _same_bits(out, ref.out) and _same_bits(lse, ref.lse)
        ref_out, ref_lse = oracle_out(w)
        check_out(out, ref_out, dtype, label="noalloc")
        check_lse(lse, ref_lse, label="noalloc")
