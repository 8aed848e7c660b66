"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every input is seeded and synthetic; pools hold NaN in every unused page and
in every slot past a row's last real token, so any read of padding shows up
as a non-finite or wrong output.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_block_amd import engine, traces
from paged_kv_gqa_block_amd._lib import PKV_ESHAPE, PkvError
from tests.parity import check_lse, check_out, oracle_out, say

pytestmark = pytest.mark.gpu

SEED = traces.HELD_OUT_SEED
PATHS = ("bucketed", "workqueue", "nosplit", "padded")
KERNELS = ("valu", "mfma")


def _applicable(kernel, d, group):
    """The matrix-core kernel covers d = 128 (any G <= 16); the vector-ALU
    kernel covers d = 64 and 128 with G <= 8."""
    return not ((kernel == "mfma" and d != 128) or (kernel == "valu" and group > 8))


def _check_rejected(w, path, splits, kernel):
    """A split kernel asked for a shape it does not cover: the decode call
    returns PKV_ESHAPE before any launch, and the stream stays usable."""
    wd = engine.to_device(w)
    step = engine.DecodeStep(engine.problem_from_workload(w, kernel), path, splits)
    step.plan(wd["seq_lens_host"])
    with pytest.raises(PkvError) as e:
        step.decode(wd)
    assert e.value.status == PKV_ESHAPE
    torch.cuda.synchronize()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    torch.cuda.init()


def _run(w, path, splits, kernel):
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    prob = engine.problem_from_workload(w, kernel)
    step = engine.DecodeStep(prob, path, splits)
    step.plan(wd["seq_lens_host"])
    step.run(wd)
    torch.cuda.synchronize()
    return step, wd


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("path", PATHS)
def test_tiny_config_all_paths(path, kernel):
    w = traces.generate(traces.get_spec("tiny"), SEED)
    if not _applicable(kernel, 64, 4):
        say(f"[tiny] path={path} kernel={kernel}: rejected shape")
        _check_rejected(w, path, w["spec"].splits, kernel)
        return
    say(f"[tiny] path={path} kernel={kernel}")
    ref_out, ref_lse = oracle_out(w)
    step, _ = _run(w, path, w["spec"].splits, kernel)
    check_out(step.out, ref_out, "f16", label=f"tiny/{path}")
    check_lse(step.lse, ref_lse, label=f"tiny/{path}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("path", ("workqueue", "bucketed", "padded"))
def test_split_states_match_oracle(path, kernel):
    d = 128 if kernel == "mfma" else 64
    spec = traces.custom_spec(3, 8, 2, d, splits=5)
    lens = np.array([200, 37, 0], dtype=np.int32)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[states] path={path} kernel={kernel}")
    step, _ = _run(w, path, 5, kernel)
    a = traces.oracle_arrays(w)
    plan = oracle.plan(lens, 2, 8, d, 16, 5, path)
    m, l, o = oracle.split_states_for_plan(a["q"], a["k_pool"], a["v_pool"], a["block_table"],
                                           plan.tasks, a["scale"], 16, "f16", 4, lens)
    gm = step.st_m.cpu().numpy().astype(np.float64)
    gl = step.st_l.cpu().numpy().astype(np.float64)
    go = step.st_o.cpu().numpy().astype(np.float64)
    for j, (row, g, s, _pb, _pe) in enumerate(plan.tasks):
        slot = j if path == "workqueue" else (row * 2 + g) * 5 + s
        lse_ref = m[j] + np.log(l[j])
        lse_got = gm[slot] + np.log(gl[slot])
        assert np.abs(lse_got - lse_ref).max() <= 2e-4, (j, lse_got, lse_ref)
        on_ref = o[j] / l[j][:, None]
        on_got = go[slot] / gl[slot][:, None]
        assert np.abs(on_got - on_ref).max() <= 1e-4, j
    if path != "workqueue":
        used = {(row * 2 + g) * 5 + s for (row, g, s, _, _) in plan.tasks}
        for slot in range(plan.n_state_slots):
            if slot not in used:
                assert np.isneginf(gm[slot]).all() and (gl[slot] == 0).all()
                assert (go[slot] == 0).all()


def test_merge_kernel_from_oracle_states():
    """The merge alone, fed with oracle states (fp64 rounded to fp32)."""
    spec = traces.custom_spec(4, 16, 2, 128, splits=7)
    lens = np.array([1000, 3, 0, 517], dtype=np.int32)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say("[merge-only]")
    a = traces.oracle_arrays(w)
    plan = oracle.plan(lens, 2, 16, 128, 16, 7, "workqueue")
    m, l, o = oracle.split_states_for_plan(a["q"], a["k_pool"], a["v_pool"], a["block_table"],
                                           plan.tasks, a["scale"], 16, "f16", 8, lens)
    wd = engine.to_device(w)
    prob = engine.problem_from_workload(w, "valu")
    step = engine.DecodeStep(prob, "workqueue", 7)
    step.plan(wd["seq_lens_host"])
    n = len(plan.tasks)
    step.st_m[:n] = torch.from_numpy(m.astype(np.float32)).cuda()
    step.st_l[:n] = torch.from_numpy(l.astype(np.float32)).cuda()
    step.st_o[:n] = torch.from_numpy(o.astype(np.float32)).cuda()
    step.merge()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_out(w)
    check_out(step.out, ref_out, "f16", label="merge-only")
    check_lse(step.lse, ref_lse, label="merge-only")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name,paths", [
    ("long", ("bucketed", "workqueue", "nosplit")),
    ("bimodal", ("workqueue", "bucketed", "nosplit", "padded")),
    ("zipf", ("workqueue", "bucketed", "nosplit", "padded")),
    ("uniform", ("workqueue", "bucketed", "nosplit", "padded")),
])
def test_full_size_configs(name, paths, kernel):
    w = traces.generate(traces.get_spec(name), SEED)
    say(f"[{name}] lens={w['seq_lens'].tolist()} kernel={kernel}")
    ref_out, ref_lse = oracle_out(w)
    for path in paths:
        say(f"  path={path}")
        step, _ = _run(w, path, w["spec"].splits, kernel)
        mx, rel = check_out(step.out, ref_out, "f16", label=f"{name}/{path}")
        check_lse(step.lse, ref_lse, label=f"{name}/{path}")
        say(f"  ok max-abs={mx:.2e} rel-l2={rel:.2e}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("batch", (1, 8))
def test_policy_sweep_slice_bf16(batch, kernel):
    w = traces.generate(traces.get_spec(f"policy_b{batch}"), SEED)
    say(f"[policy_b{batch}] kernel={kernel}")
    ref_out, ref_lse = oracle_out(w)
    for path, s in (("workqueue", 32), ("bucketed", 16), ("nosplit", 1), ("padded", 16)):
        step, _ = _run(w, path, s, kernel)
        check_out(step.out, ref_out, "bf16", label=f"policy_b{batch}/{path}")
        check_lse(step.lse, ref_lse, label=f"policy_b{batch}/{path}")


EDGE_LENS = np.array([0, 1, 15, 16, 17, 33, 100, 0, 250], dtype=np.int32)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("d", (64, 128))
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2), (6, 2), (12, 2), (32, 2)])
@pytest.mark.parametrize("dtype", ("f16", "bf16"))
def test_edge_lengths_shapes_and_dtypes(d, hq, hkv, dtype, kernel):
    spec = traces.custom_spec(len(EDGE_LENS), hq, hkv, d, splits=3, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=EDGE_LENS)
    if not _applicable(kernel, d, hq // hkv):
        say(f"[edge] d={d} hq={hq} hkv={hkv} {dtype} kernel={kernel}: rejected shape")
        for path, s in (("workqueue", 3), ("bucketed", 3), ("nosplit", 1), ("padded", 3)):
            _check_rejected(w, path, s, kernel)
        return
    say(f"[edge] d={d} hq={hq} hkv={hkv} {dtype} kernel={kernel}")
    ref_out, ref_lse = oracle_out(w)
    for path, s in (("workqueue", 3), ("workqueue", 40), ("bucketed", 3), ("bucketed", 40),
                    ("nosplit", 1), ("padded", 3), ("padded", 40)):
        step, _ = _run(w, path, s, kernel)
        check_out(step.out, ref_out, dtype, label=f"edge/{path}/S={s}")
        check_lse(step.lse, ref_lse, label=f"edge/{path}/S={s}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("path", PATHS)
def test_all_rows_empty(path, kernel):
    spec = traces.custom_spec(3, 8, 2, 128, splits=4)
    w = traces.generate(spec, SEED, seq_lens=np.zeros(3, np.int32))
    say(f"[empty] path={path}")
    step, _ = _run(w, path, 4, kernel)
    assert (step.out.float() == 0).all()
    assert torch.isneginf(step.lse).all()


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ("f16", "bf16"))
def test_single_token_gives_v_bit_exactly(dtype, kernel):
    spec = traces.custom_spec(2, 8, 2, 128, splits=4, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=np.array([1, 1], np.int32))
    say(f"[n=1] {dtype}")
    for path in PATHS:
        step, _ = _run(w, path, 4, kernel)
        bt = w["block_table"]
        for i in range(2):
            for h in range(8):
                v = w["v_pool"][bt[i, 0], h // 4, 0]
                assert torch.equal(step.out[i, h].cpu().view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("kernel", KERNELS)
def test_two_runs_are_bit_identical(kernel):
    w = traces.generate(traces.get_spec("bimodal"), SEED)
    say("[determinism]")
    s1, wd = _run(w, "workqueue", 32, kernel)
    o1 = s1.out.clone()
    s1.run(wd)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), s1.out.view(torch.int16))


@pytest.mark.parametrize("batch", (32, 64))
def test_policy_sweep_large_batches_sampled_rows(batch):
    """Full-size B=32/64 bf16 sweep workloads in the launch configuration the
    calibrated policy picks (and the four single paths); the oracle checks a
    sample of rows (first, a middle one, the longest, last)."""
    w = traces.generate(traces.get_spec(f"policy_b{batch}"), SEED)
    lens = w["seq_lens"].numpy()
    rows = sorted({0, batch // 2, int(lens.argmax()), batch - 1})
    say(f"[policy_b{batch}] sampled rows {rows}")
    ref_out, ref_lse = oracle_out(w, rows=rows)
    rules = engine.load_policy_table()
    chosen = engine.choose(rules, batch, int(lens.max()))
    for path, s in dict.fromkeys([chosen, ("workqueue", 32), ("bucketed", 32), ("nosplit", 1),
                                  ("padded", 32)]):
        step, _ = _run(w, path, s, "auto")
        check_out(step.out, ref_out, "bf16", rows=rows, label=f"policy_b{batch}/{path}:{s}")
        check_lse(step.lse, ref_lse, rows=rows, label=f"policy_b{batch}/{path}:{s}")
        assert torch.isfinite(step.out.float()).all()


@pytest.mark.parametrize("hq,hkv,dtype", [(32, 2, "bf16"), (32, 2, "f16"), (8, 8, "f16")])
def test_group_extremes_at_full_length(hq, hkv, dtype):
    """G = 16 (the two-pages-in-flight matrix-core variant) and G = 1 (plain
    multi-head decode) at long-context lengths, every path, on every row of a
    4-row batch with mixed lengths."""
    rng = np.random.default_rng(11)
    lens = np.array([32768, int(rng.integers(16385, 32768)), int(rng.integers(1, 4096)), 17],
                    dtype=np.int32)
    spec = traces.custom_spec(4, hq, hkv, 128, splits=32, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[groups] hq={hq} hkv={hkv} {dtype} lens={lens.tolist()}")
    ref_out, ref_lse = oracle_out(w)
    for path, s in (("workqueue", 32), ("bucketed", 32), ("padded", 32), ("nosplit", 1)):
        step, _ = _run(w, path, s, "auto")
        check_out(step.out, ref_out, dtype, label=f"groups/{hq}/{hkv}/{path}")
        check_lse(step.lse, ref_lse, label=f"groups/{hq}/{hkv}/{path}")


@pytest.mark.parametrize("seed", range(24))
def test_random_small_problems_every_path(seed):
    """Random shapes, dtypes, split caps and lengths (with the page-boundary
    values mixed in), every path and the kernel AUTO picks, element by element
    against the oracle."""
    rng = np.random.default_rng(4000 + seed)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8] + ([16] if d == 128 else [])))
    b = int(rng.integers(1, 7))
    dtype = str(rng.choice(["f16", "bf16"]))
    lens = rng.integers(0, 1200, size=b)
    edge = rng.choice([0, 1, 15, 16, 17, 31, 32, 33], size=b)
    lens = np.where(rng.random(b) < 0.4, edge, lens).astype(np.int32)
    s = int(rng.choice([1, 2, 3, 5, 8, 32, 100]))
    spec = traces.custom_spec(b, hkv * g, hkv, d, splits=s, dtype=dtype)
    w = traces.generate(spec, SEED + seed, seq_lens=lens)
    say(f"[random {seed}] B={b} Hq={hkv * g} Hkv={hkv} d={d} {dtype} S={s} lens={lens.tolist()}")
    ref_out, ref_lse = oracle_out(w)
    for path in PATHS:
        step, _ = _run(w, path, 1 if path == "nosplit" else s, "auto")
        check_out(step.out, ref_out, dtype, label=f"random{seed}/{path}")
        check_lse(step.lse, ref_lse, label=f"random{seed}/{path}")


@pytest.mark.parametrize("lens", ([500, 510, 497, 512],    # equal page counts
                                  [481, 512, 465, 450],    # equal split counts, unequal pages
                                  [481, 512, 0, 450],      # an empty row: counts differ
                                  [481, 512, 40, 450]))    # a short row: counts differ
def test_workqueue_merge_with_shared_and_mixed_split_counts(lens):
    """The workqueue merge locates a row's states from its index when every
    row has the same split count, and from the plan's row arrays otherwise:
    both against the oracle, on both kernels' states.  With a shared split
    count (B * Hkv = 32 pairs) the split launch also takes its XCD-affine
    task order."""
    lens = np.asarray(lens, dtype=np.int32)
    spec = traces.custom_spec(4, 32, 8, 128, splits=8, dtype="f16")
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[wq merge] lens={lens.tolist()}")
    ref_out, ref_lse = oracle_out(w)
    for kernel in KERNELS:
        step, _ = _run(w, "workqueue", 8, kernel)
        check_out(step.out, ref_out, "f16", label=f"wqmerge/{kernel}")
        check_lse(step.lse, ref_lse, label=f"wqmerge/{kernel}")


def test_large_batch_short_contexts_every_path():
    """512 rows of 1..600 tokens (G = 8, bf16): hundreds of exact buckets and
    grids of tens of thousands of workgroups, on sampled rows."""
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 601, size=512).astype(np.int32)
    lens[::97] = 0
    spec = traces.custom_spec(512, 64, 8, 128, splits=8, dtype="bf16")
    w = traces.generate(spec, SEED, seq_lens=lens)
    rows = sorted({0, 1, 97, 255, int(lens.argmax()), 510, 511})
    say(f"[large batch] B=512 rows {rows}")
    ref_out, ref_lse = oracle_out(w, rows=rows)
    for path, s in (("workqueue", 8), ("bucketed", 8), ("padded", 8), ("nosplit", 1)):
        step, _ = _run(w, path, s, "auto")
        check_out(step.out, ref_out, "bf16", rows=rows, label=f"large/{path}")
        check_lse(step.lse, ref_lse, rows=rows, label=f"large/{path}")
        assert torch.isfinite(step.out.float()).all()


@pytest.mark.parametrize("hq,hkv,b,n", [(16, 4, 2, 700), (8, 1, 8, 333), (32, 8, 3, 1000)])
def test_workqueue_xcd_launch_order(hq, hkv, b, n):
    """Equal lengths give every row the same split count, and B * Hkv is a
    multiple of 8 (8, 8 and 24 pairs), so the split launch takes its
    XCD-affine task order (a permutation of the tasks over the blocks).  With
    Hkv = 4 or 1 a KV head's splits and its merge sit on different XCDs, which
    changes nothing in the results: every case matches the oracle on both
    kernels."""
    lens = np.full(b, n, dtype=np.int32)
    spec = traces.custom_spec(b, hq, hkv, 128, splits=16, dtype="bf16")
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[wq xcd] hq={hq} hkv={hkv} b={b} n={n}")
    ref_out, ref_lse = oracle_out(w)
    for kernel in KERNELS:
        step, _ = _run(w, "workqueue", 16, kernel)
        check_out(step.out, ref_out, "bf16", label=f"wqxcd/{kernel}")
        check_lse(step.lse, ref_lse, label=f"wqxcd/{kernel}")


@pytest.mark.parametrize("seed", range(10))
def test_random_equal_split_counts_every_split_path(seed):
    """Random head shapes, batch sizes, split caps and dtypes with lengths
    drawn so that every row gets the same split count: the workqueue launch
    takes its XCD-affine order whenever B * Hkv is a multiple of 8, and bucket
    launches their (KV head, split, row) grid.  Every split path on both
    kernels against the oracle."""
    rng = np.random.default_rng(7100 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    b = int(rng.choice([1, 2, 4, 8, 16])) if seed % 2 == 0 else int(rng.integers(1, 17))
    dtype = str(rng.choice(["f16", "bf16"]))
    splits = int(rng.choice([2, 5, 8, 16, 32]))
    tmax = int(rng.integers(1, 200))  # pages of the longest row
    pps = max(1, -(-tmax // splits))  # the batch-shared granule
    ns = -(-tmax // pps)
    pages = rng.integers((ns - 1) * pps + 1, tmax + 1, size=b)
    pages[0] = tmax
    lens = ((pages - 1) * 16 + rng.integers(1, 17, size=b)).astype(np.int32)
    spec = traces.custom_spec(b, hkv * g, hkv, 128, splits=splits, dtype=dtype)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[equal splits {seed}] B={b} Hq={hkv * g} Hkv={hkv} S={splits} ns={ns} {dtype}")
    ref_out, ref_lse = oracle_out(w)
    for kernel in KERNELS:
        for path in ("workqueue", "bucketed", "padded"):
            step, _ = _run(w, path, splits, kernel)
            check_out(step.out, ref_out, dtype, label=f"equal{seed}/{kernel}/{path}")
            check_lse(step.lse, ref_lse, label=f"equal{seed}/{kernel}/{path}")


def _peaked(w, q_scale, targets):
    """Sharply peaked scores.  q is multiplied by q_scale (a typical score then
    has standard deviation q_scale), and for every row and KV head g the key of
    a few planted tokens is set so that the score of query head g * G is
    targets[k] (up to the 16-bit rounding of the key): the planted tokens lie in
    different splits, the largest one late in its split (its page raises the
    running maximum by a wide margin), and the other splits' maxima sit tens of
    natural-log units below the row maximum (their weights underflow)."""
    spec = w["spec"]
    dt = w["q"].dtype
    q = (w["q"].float() * q_scale).to(dt)
    k_pool = w["k_pool"].clone()
    bt = w["block_table"].numpy()
    grp = spec.group
    for i, n in enumerate(w["seq_lens"].numpy()):
        n = int(n)
        if n == 0:
            continue
        spots = [min(n - 1, int(f * n)) for f in (0.62, 0.15, 0.97)][:len(targets)]
        for k, (t, target) in enumerate(zip(spots, targets)):
            page, slot = int(bt[i, t // spec.page_size]), t % spec.page_size
            for g in range(spec.num_kv_heads):
                qh = q[i, g * grp].double()
                key = qh * (target / w["scale"] / float(qh @ qh))
                k_pool[page, g, slot] = key.to(dt)
    return dict(w, q=q, k_pool=k_pool)


@pytest.mark.parametrize("dtype", ("f16", "bf16"))
@pytest.mark.parametrize("regime,q_scale,targets", [
    ("spread", 12.0, (60.0, 58.0, 55.0)),    # P spans fp16's subnormal range
    ("extreme", 4.0, (200.0, 199.0, 120.0)),  # every other split underflows
])
def test_peaked_softmax_every_path(regime, q_scale, targets, dtype):
    """Scores spanning about +-50 to +-200 natural-log units: one or a few
    tokens in different splits dominate, the merge weights of the other splits
    underflow, the running maximum grows by a wide margin inside a split, and
    in the spread regime the P values of a split reach fp16's subnormal range.
    Every path and both kernels, fp16 and bf16, against the oracle."""
    lens = np.array([32768, 5000, 777, 0], dtype=np.int32)
    spec = traces.custom_spec(4, 32, 8, 128, splits=32, dtype=dtype)
    w = _peaked(traces.generate(spec, SEED, seq_lens=lens), q_scale, targets)
    say(f"[peaked {regime}] {dtype} q_scale={q_scale} targets={targets}")
    ref_out, ref_lse = oracle_out(w)
    assert np.abs(ref_out).max() > 0.5  # outputs dominated by a few V rows
    for kernel in KERNELS:
        for path, s in (("workqueue", 32), ("bucketed", 32), ("padded", 32), ("nosplit", 1),
                        ("workqueue", 7)):
            step, _ = _run(w, path, s, kernel)
            check_out(step.out, ref_out, dtype, label=f"peaked/{regime}/{kernel}/{path}:{s}")
            check_lse(step.lse, ref_lse, label=f"peaked/{regime}/{kernel}/{path}:{s}")


@pytest.mark.parametrize("name", ("long", "bimodal", "zipf", "uniform", "tiny", "policy_b1",
                                  "policy_b8", "policy_short_b4", "policy_short_b16",
                                  "policy_b32"))
def test_cost_model_choice_matches_oracle(name):
    """The learned cost model's choice (pkv_policy_model with the weights of
    the problem's split kernel) run through the C ABI on the trace and sweep
    workloads, against the oracle (B = 32 on sampled rows)."""
    w = traces.generate(traces.get_spec(name), SEED)
    spec = w["spec"]
    lens = w["seq_lens"].numpy()
    path, s, pred = engine.choose_model(engine.load_cost_model(),
                                        engine.problem_from_workload(w), lens)
    rows = None if spec.batch <= 16 else sorted({0, spec.batch // 2, int(lens.argmax()),
                                                 spec.batch - 1})
    say(f"[cost model {name}] choice {path}:{s} predicted {pred:.1f} us rows={rows}")
    ref_out, ref_lse = oracle_out(w, rows=rows)
    step, _ = _run(w, path, s, "auto")
    check_out(step.out, ref_out, spec.dtype, rows=rows, label=f"model/{name}/{path}:{s}")
    check_lse(step.lse, ref_lse, rows=rows, label=f"model/{name}/{path}:{s}")


@pytest.mark.parametrize("name", ("bimodal", "zipf", "uniform", "policy_b4", "policy_b8",
                                  "policy_short_b8", "policy_short_b16"))
def test_default_policy_choice_matches_oracle(name):
    """The engine's default choice (pkv_policy_default), which on these
    workloads is the workqueue at a CU-balanced split cap outside the listed
    8/16/32/64 (e.g. 15 on bimodal, 3 on the short B = 16 sweep), run through
    the C ABI against the oracle."""
    w = traces.generate(traces.get_spec(name), SEED)
    spec = w["spec"]
    lens = w["seq_lens"].numpy()
    path, s = engine.choose_default(engine.load_policy_table(), engine.load_cost_model(),
                                    engine.problem_from_workload(w), lens)
    say(f"[default policy {name}] choice {path}:{s}")
    ref_out, ref_lse = oracle_out(w)
    step, _ = _run(w, path, s, "auto")
    check_out(step.out, ref_out, spec.dtype, label=f"default/{name}/{path}:{s}")
    check_lse(step.lse, ref_lse, label=f"default/{name}/{path}:{s}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_nosplit_takes_row_lengths_from_the_plan(kernel):
    """pkv_decode reads every row's length from the plan on every path: on the
    no-split path a device length array that disagrees with the plan (here
    each entry within the row's table capacity, so any read stays in bounds)
    changes nothing; the output matches the oracle at the planned lengths."""
    from paged_kv_gqa_block_amd import _lib

    d = 128 if kernel == "mfma" else 64
    lens = np.array([300, 17, 0], dtype=np.int32)
    spec = traces.custom_spec(3, 8, 2, d, splits=4)
    w = traces.generate(spec, SEED, seq_lens=lens)
    say(f"[nosplit plan lengths] kernel={kernel}")
    wd = engine.to_device(w)
    engine.validate_inputs(wd)
    step = engine.DecodeStep(engine.problem_from_workload(w, kernel), "nosplit", 1)
    step.plan(wd["seq_lens_host"])
    stale = torch.tensor([17, 300, 250], dtype=torch.int32, device="cuda")
    _lib.pkv_decode(step.prob, step.plan_host, step.plan_dev, wd["q"], wd["k_pool"],
                    wd["v_pool"], wd["block_table"], stale, None, None, None, step.out, step.lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_out(w)
    check_out(step.out, ref_out, "f16", label="nosplit/plan lengths")
    check_lse(step.lse, ref_lse, label="nosplit/plan lengths")
