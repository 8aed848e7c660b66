"""Pins for the fp64 attention oracle (CPU only).

Each pin ties the oracle to something other than itself: torch's dense
scaled-dot-product attention, closed forms, a hand-worked example, and
invariants that a dropped term, a wrong sign, a wrong index or a transposed
operand would break.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention, merge, split_state

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paged_from_dense(k_dense, v_dense, lens, page_size, rng, extra_pages=3):
    """Scatter dense [B][Hkv][Nmax][d] K/V into a shuffled pool; NaN elsewhere."""
    b, hkv, _, d = k_dense.shape
    pages = [-(-int(n) // page_size) for n in lens]
    used = sum(pages)
    pool = used + extra_pages
    perm = rng.permutation(pool)
    k_pool = np.full((pool, hkv, page_size, d), np.nan, dtype=np.float16)
    v_pool = np.full_like(k_pool, np.nan)
    bt = np.full((b, max(1, max(pages))), perm[-1], dtype=np.int32)
    off = 0
    for i, n in enumerate(lens):
        bt[i, :pages[i]] = perm[off:off + pages[i]]
        off += pages[i]
        for t in range(int(n)):
            k_pool[bt[i, t // page_size], :, t % page_size] = k_dense[i, :, t]
            v_pool[bt[i, t // page_size], :, t % page_size] = v_dense[i, :, t]
    return k_pool, v_pool, bt


def _random_case(rng, b, hq, hkv, d, lens, page_size):
    nmax = max(1, max(lens))
    q = rng.standard_normal((b, hq, d)).astype(np.float16)
    kd = rng.standard_normal((b, hkv, nmax, d)).astype(np.float16)
    vd = rng.standard_normal((b, hkv, nmax, d)).astype(np.float16)
    k_pool, v_pool, bt = _paged_from_dense(kd, vd, lens, page_size, rng)
    return q, kd, vd, k_pool, v_pool, bt


@pytest.mark.parametrize("hq,hkv,d,lens,page_size", [
    (8, 2, 16, [37, 1, 16, 0], 4),
    (4, 4, 8, [5, 12], 4),      # G = 1: textbook multi-head decode
    (6, 1, 8, [33], 16),        # G = 6, a single KV head
    (8, 2, 64, [100, 17, 64], 16),
])
def test_attention_matches_torch_sdpa_on_dense_kv(hq, hkv, d, lens, page_size):
    rng = np.random.default_rng(7)
    b = len(lens)
    q, kd, vd, k_pool, v_pool, bt = _random_case(rng, b, hq, hkv, d, lens, page_size)
    scale = 1.0 / math.sqrt(d)
    out, lse = attention(q, k_pool, v_pool, bt, np.array(lens), scale, page_size, "f16")
    for i, n in enumerate(lens):
        if n == 0:
            assert np.all(out[i] == 0) and np.all(np.isneginf(lse[i]))
            continue
        qt = torch.from_numpy(q[i].astype(np.float64))[None, :, None, :]    # [1,Hq,1,d]
        kt = torch.from_numpy(kd[i, :, :n].astype(np.float64))[None]        # [1,Hkv,n,d]
        vt = torch.from_numpy(vd[i, :, :n].astype(np.float64))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=scale, enable_gqa=True)[0, :, 0].numpy()
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)
        # lse against torch.logsumexp of the scores, KV heads expanded by torch.
        kx = kt.repeat_interleave(hq // hkv, dim=1)[0]                      # [Hq,n,d]
        scores = torch.einsum("hd,hnd->hn", qt[0, :, 0], kx) * scale
        np.testing.assert_allclose(lse[i], torch.logsumexp(scores, dim=-1).numpy(),
                                   rtol=1e-12, atol=1e-12)


def _brute_force_row_head(q, k_pool, v_pool, bt_row, n, h, group, scale, page_size):
    """Scalar loops over Python floats: the decode definition, token by token."""
    g = h // group
    scores, vals = [], []
    for t in range(n):
        page, slot = int(bt_row[t // page_size]), t % page_size
        k = [float(x) for x in k_pool[page, g, slot]]
        v = [float(x) for x in v_pool[page, g, slot]]
        scores.append(scale * sum(float(a) * b for a, b in zip(q[h], k)))
        vals.append(v)
    if n == 0:
        return [0.0] * q.shape[-1], -math.inf
    mx = max(scores)
    w = [math.exp(x - mx) for x in scores]
    den = sum(w)
    out = [sum(w[t] * vals[t][j] for t in range(n)) / den for j in range(q.shape[-1])]
    return out, mx + math.log(den)


@pytest.mark.parametrize("seed", range(6))
def test_attention_matches_scalar_brute_force_on_tiny_shapes(seed):
    """B <= 3, N <= 40 with the page-boundary lengths, d = 8, P = 4."""
    rng = np.random.default_rng(300 + seed)
    b = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 3]))
    lens = [int(x) for x in rng.choice([0, 1, 3, 4, 5, 8, 9, 17, 40], size=b)]
    q, _, _, k_pool, v_pool, bt = _random_case(rng, b, hq, hkv, 8, lens, 4)
    scale = 1.0 / math.sqrt(8)
    out, lse = attention(q, k_pool, v_pool, bt, np.array(lens), scale, 4, "f16")
    for i, n in enumerate(lens):
        for h in range(hq):
            ref, ref_lse = _brute_force_row_head(q[i], k_pool, v_pool, bt[i], n, h, hq // hkv,
                                                 scale, 4)
            np.testing.assert_allclose(out[i, h], ref, rtol=1e-12, atol=1e-12)
            if n == 0:
                assert math.isinf(lse[i, h]) and lse[i, h] < 0
            else:
                assert abs(lse[i, h] - ref_lse) <= 1e-12 * max(1.0, abs(ref_lse))


def test_golden_two_token_example():
    with open(os.path.join(GOLDEN, "two_token_example.json")) as f:
        g = json.load(f)

    def arr(x):
        return np.array(x, dtype=np.float64).astype(np.float16)

    out, lse = attention(arr(g["q"]), arr(g["k_pool"]), arr(g["v_pool"]),
                         np.array(g["block_table"], dtype=np.int32),
                         np.array(g["seq_lens"]), g["scale"], g["page_size"], "f16")
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), rtol=0, atol=1e-12)


def test_single_token_gives_v_exactly():
    rng = np.random.default_rng(1)
    q, kd, vd, k_pool, v_pool, bt = _random_case(rng, 2, 4, 2, 32, [1, 1], 16)
    out, lse = attention(q, k_pool, v_pool, bt, np.array([1, 1]), 0.125, 16, "f16")
    for i in range(2):
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[i, h], vd[i, g, 0].astype(np.float64))
            assert lse[i, h] == pytest.approx(
                0.125 * float(np.dot(q[i, h].astype(np.float64), kd[i, g, 0].astype(np.float64))),
                abs=1e-12)


def test_constant_keys_and_zero_query_give_mean_of_v():
    rng = np.random.default_rng(2)
    n, d = 45, 16
    q, kd, vd, k_pool, v_pool, bt = _random_case(rng, 1, 2, 1, d, [n], 8)
    # Constant keys: every token gets the same score -> uniform weights.
    kd_const = np.repeat(kd[:, :, :1], n, axis=2)
    k_pool_c, v_pool_c, bt_c = _paged_from_dense(kd_const, vd, [n], 8, rng)
    out, lse = attention(q, k_pool_c, v_pool_c, bt_c, np.array([n]), 0.25, 8, "f16")
    mean_v = vd[0, 0, :n].astype(np.float64).mean(axis=0)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], mean_v, rtol=1e-12, atol=1e-12)
        x = 0.25 * float(q[0, h].astype(np.float64) @ kd[0, 0, 0].astype(np.float64))
        assert lse[0, h] == pytest.approx(x + math.log(n), abs=1e-12)
    # Zero query: all scores are 0 -> mean of V, lse = ln N.
    q0 = np.zeros_like(q)
    out0, lse0 = attention(q0, k_pool, v_pool, bt, np.array([n]), 0.25, 8, "f16")
    np.testing.assert_allclose(out0[0, 0], mean_v, rtol=1e-12, atol=1e-12)
    assert lse0[0, 0] == pytest.approx(math.log(n), abs=1e-12)


def test_block_table_permutation_invariance_is_bit_exact():
    rng = np.random.default_rng(3)
    lens = [50, 7, 33]
    q, _, _, k_pool, v_pool, bt = _random_case(rng, 3, 4, 2, 16, lens, 8)
    out, lse = attention(q, k_pool, v_pool, bt, np.array(lens), 0.3, 8, "f16")
    perm = rng.permutation(k_pool.shape[0])  # new page id of old page p is perm[p]
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[perm] = k_pool
    v2[perm] = v_pool
    out2, lse2 = attention(q, k2, v2, perm[bt].astype(np.int32), np.array(lens), 0.3, 8, "f16")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_score_shift_and_linearity_in_v():
    rng = np.random.default_rng(4)
    n, d = 29, 8
    q = rng.integers(-3, 4, size=(1, 2, d)).astype(np.float16)
    kd = rng.integers(-3, 4, size=(1, 1, n, d)).astype(np.float16)
    u = rng.integers(-2, 3, size=d).astype(np.float16)
    v1 = rng.integers(-5, 6, size=(1, 1, n, d)).astype(np.float16)
    v2 = rng.integers(-5, 6, size=(1, 1, n, d)).astype(np.float16)
    scale = 0.1

    def run(k, v):
        kp, vp, bt = _paged_from_dense(k, v, [n], 4, np.random.default_rng(0))
        return attention(q, kp, vp, bt, np.array([n]), scale, 4, "f16")

    out_a, lse_a = run(kd, v1)
    # Adding the same vector u to every key shifts all scores of a head by
    # scale * <q_h, u>: the output is unchanged and the lse moves by that shift.
    out_b, lse_b = run((kd.astype(np.float64) + u).astype(np.float16), v1)
    np.testing.assert_allclose(out_b, out_a, rtol=1e-12, atol=1e-12)
    shift = scale * (q[0].astype(np.float64) @ u.astype(np.float64))
    np.testing.assert_allclose(lse_b[0], lse_a[0] + shift, rtol=0, atol=1e-12)
    # Output is linear in V.
    out_2, _ = run(kd, v2)
    out_s, _ = run(kd, (v1.astype(np.float64) + v2).astype(np.float16))
    np.testing.assert_allclose(out_s, out_a + out_2, rtol=1e-12, atol=1e-12)


def test_split_then_merge_equals_unsplit():
    rng = np.random.default_rng(5)
    lens = [123]
    hq, hkv, d, p = 8, 2, 16, 8
    q, _, _, k_pool, v_pool, bt = _random_case(rng, 1, hq, hkv, d, lens, p)
    out, lse = attention(q, k_pool, v_pool, bt, np.array(lens), 0.25, p, "f16")
    grp = hq // hkv
    for trial in range(6):
        cuts = sorted(rng.choice(np.arange(1, 123), size=trial, replace=False).tolist())
        bounds = [0] + cuts + [123]
        for g in range(hkv):
            states = [split_state(q, k_pool, v_pool, bt[0], 0, g, a, b, 0.25, p, "f16", grp)
                      for a, b in zip(bounds[:-1], bounds[1:])]
            # Add neutral (empty) states and shuffle the order: neither may matter.
            states.append(split_state(q, k_pool, v_pool, bt[0], 0, g, 50, 50, 0.25, p, "f16", grp))
            order = rng.permutation(len(states))
            ms = np.stack([states[j][0] for j in order])
            ls = np.stack([states[j][1] for j in order])
            os_ = np.stack([states[j][2] for j in order])
            o_m, l_m = merge(ms, ls, os_)
            np.testing.assert_allclose(o_m, out[0, g * grp:(g + 1) * grp], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(l_m, lse[0, g * grp:(g + 1) * grp], rtol=1e-12, atol=1e-12)


def test_single_split_state_normalises_to_unsplit():
    rng = np.random.default_rng(6)
    q, _, _, k_pool, v_pool, bt = _random_case(rng, 1, 4, 1, 16, [40], 16)
    out, lse = attention(q, k_pool, v_pool, bt, np.array([40]), 0.25, 16, "f16")
    m, l, o = split_state(q, k_pool, v_pool, bt[0], 0, 0, 0, 40, 0.25, 16, "f16", 4)
    np.testing.assert_allclose(o / l[:, None], out[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m + np.log(l), lse[0], rtol=1e-12, atol=1e-12)


def test_all_neutral_merge_gives_zero_and_neg_inf():
    ms = np.full((3, 2), -np.inf)
    ls = np.zeros((3, 2))
    os_ = np.zeros((3, 2, 4))
    out, lse = merge(ms, ls, os_)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_empty_split_state_is_neutral():
    rng = np.random.default_rng(8)
    q, _, _, k_pool, v_pool, bt = _random_case(rng, 1, 2, 1, 8, [10], 4)
    m, l, o = split_state(q, k_pool, v_pool, bt[0], 0, 0, 8, 8, 1.0, 4, "f16", 2)
    assert np.all(np.isneginf(m)) and np.all(l == 0) and np.all(o == 0)


def test_bf16_decode_and_rounding_match_torch():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, size=4096)).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.decode_values(bits, "bf16"),
                                  t.to(torch.float64).numpy())
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)),
                                  t.to(torch.float64).numpy())
    np.testing.assert_array_equal(oracle.round_to_f16(x.astype(np.float64)),
                                  torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy())


def test_bf16_path_matches_f16_path_on_shared_values():
    """Values exactly representable in both formats give identical results."""
    rng = np.random.default_rng(10)
    lens = [21, 3]
    q = rng.integers(-4, 5, size=(2, 4, 8)).astype(np.float16)
    kd = rng.integers(-4, 5, size=(2, 2, 21, 8)).astype(np.float16)
    vd = rng.integers(-4, 5, size=(2, 2, 21, 8)).astype(np.float16)
    kp, vp, bt = _paged_from_dense(kd, vd, lens, 4, rng)

    def to_bf16_bits(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)

    o1, l1 = attention(q, kp, vp, bt, np.array(lens), 0.5, 4, "f16")
    o2, l2 = attention(to_bf16_bits(q), to_bf16_bits(kp), to_bf16_bits(vp), bt, np.array(lens),
                       0.5, 4, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_append_oracle_writes_only_the_addressed_slot():
    rng = np.random.default_rng(11)
    pool = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    v_pool = rng.standard_normal((6, 2, 4, 8)).astype(np.float16)
    bt = np.array([[5, 2], [1, 0]], dtype=np.int32)
    k_new = rng.standard_normal((2, 2, 8)).astype(np.float16)
    v_new = rng.standard_normal((2, 2, 8)).astype(np.float16)
    k2, v2 = oracle.append_kv(pool, v_pool, bt, np.array([6, -1]), k_new, v_new, 4)
    # Position 6 of row 0 = page bt[0][1] = 2, slot 2; row 1 is inactive.
    assert np.array_equal(k2[2, :, 2], k_new[0]) and np.array_equal(v2[2, :, 2], v_new[0])
    mask = np.ones(k2.shape[:3], bool)
    mask[2, :, 2] = False
    assert np.array_equal(k2[mask], pool[mask]) and np.array_equal(v2[mask], v_pool[mask])


def test_append_one_by_one_rebuilds_the_dense_sequence():
    """Appending tokens 0..N-1 in order reproduces the dense K/V through the table."""
    rng = np.random.default_rng(12)
    n, hkv, d, p = 13, 2, 8, 4
    kd = rng.standard_normal((n, hkv, d)).astype(np.float16)
    vd = rng.standard_normal((n, hkv, d)).astype(np.float16)
    bt = np.array([[3, 0, 4, 1]], dtype=np.int32)
    k = np.full((5, hkv, p, d), np.nan, np.float16)
    v = np.full_like(k, np.nan)
    for t in range(n):
        k, v = oracle.append_kv(k, v, bt, np.array([t]), kd[t][None], vd[t][None], p)
    got_k, got_v = oracle.gather_row(k, v, bt[0], n, 1, p, "f16")
    np.testing.assert_array_equal(got_k, kd[:, 1].astype(np.float64))
    np.testing.assert_array_equal(got_v, vd[:, 1].astype(np.float64))


@pytest.mark.parametrize("path", ["workqueue", "bucketed", "padded", "nosplit"])
@pytest.mark.parametrize("seed", range(4))
def test_plan_task_states_merge_to_unsplit_attention(path, seed):
    """oracle.split_states_for_plan over every task of oracle.plan, merged per
    (row, KV head), equals oracle.attention: the tasks cover each row's real
    tokens exactly once (lengths off page boundaries, rows shorter than the
    split cap, an empty row), and each task reads only its own token range
    (page tails hold NaN)."""
    rng = np.random.default_rng(4100 + seed)
    page = int(rng.choice([4, 16]))
    lens = [int(x) for x in rng.choice([0, 1, page - 1, page, page + 1, 3 * page + 2, 57, 200],
                                       size=5)]
    lens[int(rng.integers(0, 5))] = 0
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 3, 4]))
    splits = int(rng.choice([1, 3, 8, 64]))
    d = 16
    q, _, _, k_pool, v_pool, bt = _random_case(rng, len(lens), hq, hkv, d, lens, page)
    scale = 1.0 / math.sqrt(d)
    ref, ref_lse = attention(q, k_pool, v_pool, bt, np.array(lens), scale, page, "f16")
    p = oracle.plan(lens, hkv, hq, d, page, splits, path)
    grp = hq // hkv
    m, l, o = oracle.split_states_for_plan(q, k_pool, v_pool, bt, p.tasks, scale, page, "f16",
                                           grp, lens)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    for i, n in enumerate(lens):
        for g in range(hkv):
            idx = [j for j, t in enumerate(p.tasks) if t[0] == i and t[1] == g]
            if n == 0:
                assert not idx
                continue
            out, lse = merge(m[idx], l[idx], o[idx])
            np.testing.assert_allclose(out, ref[i, g * grp:(g + 1) * grp], rtol=1e-12,
                                       atol=1e-12)
            np.testing.assert_allclose(lse, ref_lse[i, g * grp:(g + 1) * grp], rtol=1e-12,
                                       atol=1e-12)
