"""The seeded workload generator: determinism, shapes, length laws, NaN poisoning."""
import numpy as np
import torch

from paged_kv_gqa_block_amd import traces


def test_deterministic_and_shaped():
    a = traces.generate(traces.get_spec("tiny"), 20260623)
    b = traces.generate(traces.get_spec("tiny"), 20260623)
    for key in ("q", "k_pool", "v_pool", "block_table", "seq_lens"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].is_floating_point() else a[key],
                           b[key].view(torch.uint8) if b[key].is_floating_point() else b[key])
    assert a["q"].shape == (1, 8, 64) and a["q"].dtype == torch.float16
    assert a["k_pool"].shape == (256, 2, 16, 64)
    assert a["block_table"].shape == (1, 128)
    assert a["seq_lens"].tolist() == [2048]
    assert a["scale"] == float(np.float32(0.125))


def test_rows_use_disjoint_pages_and_unused_pages_are_nan():
    w = traces.generate(traces.get_spec("bimodal"), 20260623)
    lens = w["seq_lens"].numpy()
    bt = w["block_table"].numpy()
    used = []
    for i, n in enumerate(lens):
        used.extend(bt[i, :(-(-int(n) // 16))].tolist())
    assert len(used) == len(set(used))
    pool = w["num_pool_pages"]
    assert pool == (3 * len(used) + 1) // 2
    unused = sorted(set(range(pool)) - set(used))
    assert torch.isnan(w["k_pool"][unused].float()).all()
    assert torch.isnan(w["v_pool"][unused].float()).all()
    assert not torch.isnan(w["k_pool"][used].float()[:, :, :1]).any()
    # Tails past each row's last real token are NaN; padding entries point at NaN pages.
    for i, n in enumerate(lens):
        t = -(-int(n) // 16)
        tail = int(n) - (t - 1) * 16
        if tail < 16:
            assert torch.isnan(w["k_pool"][bt[i, t - 1], :, tail:].float()).all()
        if t < bt.shape[1]:
            assert bt[i, t] in unused


def test_length_laws():
    rng_lens = traces.draw_lengths(traces.get_spec("bimodal"), np.random.default_rng(1))
    assert sorted((rng_lens < 4096).tolist()).count(True) == 4
    assert all(128 <= n <= 2048 or 16384 <= n <= 32768 for n in rng_lens)
    z = traces.draw_lengths(traces.get_spec("zipf", batch=4000), np.random.default_rng(2))
    assert z.min() >= 64 and z.max() <= 32768 and np.all(z % 64 == 0)
    assert 0.12 < np.mean(z == 64) < 0.24  # P(k=1) of Zipf(1.2) is 1/zeta(1.2) ~ 0.18
    u = traces.draw_lengths(traces.get_spec("policy_b64"), np.random.default_rng(3))
    assert u.min() >= 1024 and u.max() <= 32768
    assert traces.get_spec("policy_b64").dtype == "bf16"


def test_bf16_oracle_encoding_roundtrips():
    w = traces.generate(traces.get_spec("policy_b1"), 20260622, seq_lens=np.array([40]))
    arrs = traces.oracle_arrays(w)
    assert arrs["q"].dtype == np.uint16
    back = torch.from_numpy(arrs["q"].view(np.int16)).view(torch.bfloat16)
    assert torch.equal(back.view(torch.int16), w["q"].view(torch.int16))
