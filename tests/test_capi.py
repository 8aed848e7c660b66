"""C-ABI tests that need no GPU: exports, host planner vs the planner oracle,
policy vs the policy oracle, and argument validation (nothing is launched)."""
import os
import re

import numpy as np
import pytest

from oracle.planner import plan as oracle_plan
from oracle.policy import choose as oracle_choose
from paged_kv_gqa_block_amd import _lib
from paged_kv_gqa_block_amd._lib import (PKV_BUCKETED, PKV_EDTYPE, PKV_EINVAL, PKV_ENOSPC,
                                         PKV_ERANGE, PKV_ESHAPE, PKV_NOSPLIT, PKV_PADDED,
                                         PKV_WORKQUEUE, PATH_NAMES, PkvError)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pkv.h")


def test_library_exports_every_declared_symbol():
    with open(HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(pkv_\w+)\s*\(", text, flags=re.M))
    assert {"pkv_plan", "pkv_decode", "pkv_merge", "pkv_policy"} <= declared
    for name in sorted(declared):
        assert hasattr(_lib.LIB, name), name
    assert set(_lib.EXPORTED) == declared


def _prob(b, hq=32, hkv=8, d=128, max_pages=2048, dtype="f16", pool=4096):
    return _lib.make_problem(b, hq, hkv, d, 16, pool, max_pages, dtype)


def _plan(prob, lens, path, s):
    nbytes = _lib.pkv_plan_bytes(prob, path, s)
    buf = np.zeros(nbytes // 4, dtype=np.int32)
    info = _lib.pkv_plan(prob, np.asarray(lens, dtype=np.int32), path, s, buf)
    return info, _lib.decode_plan(buf)


@pytest.mark.parametrize("seed", range(25))
@pytest.mark.parametrize("path", [PKV_WORKQUEUE, PKV_BUCKETED, PKV_NOSPLIT, PKV_PADDED])
def test_host_planner_matches_oracle_bit_exactly(seed, path):
    rng = np.random.default_rng(1000 + seed)
    b = int(rng.integers(1, 17))
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8]))
    s = int(rng.choice([1, 2, 4, 7, 32, 64]))
    kind = seed % 3
    if kind == 0:
        lens = rng.integers(0, 32768, size=b, endpoint=True)
    elif kind == 1:  # many repeated lengths -> few buckets
        lens = rng.choice([0, 1, 16, 17, 4096, 32768], size=b)
    else:
        lens = np.concatenate([rng.integers(128, 2048, b // 2, endpoint=True),
                               rng.integers(16384, 32768, b - b // 2, endpoint=True)])
    prob = _prob(b, hq=hkv * g, hkv=hkv)
    info, got = _plan(prob, lens, path, s)
    ref = oracle_plan(lens, hkv, hkv * g, 128, 16, s, PATH_NAMES[path])
    assert got["tasks"] == ref.tasks
    assert got["row_pages"] == ref.row_pages
    assert got["row_nsplit"] == ref.row_nsplit
    assert got["row_len"] == [int(x) for x in lens]
    if path == PKV_WORKQUEUE:
        assert got["row_task_off"] == ref.row_task_off
        assert got["pages_per_split"] == ref.pages_per_split
    if path in (PKV_BUCKETED, PKV_PADDED):
        assert [(bk[0], bk[1], bk[2], bk[3], bk[4]) for bk in got["buckets"]] == [
            (r[0], r[1], r[2], r[3], len(r[4])) for r in ref.buckets]
        rows = []
        for r in ref.buckets:
            rows.extend(r[4])
        assert got["bucket_rows"] == rows
    assert info.n_tasks == len(ref.tasks)
    assert info.n_launches == ref.n_launches
    assert info.n_state_slots == ref.n_state_slots
    assert info.n_empty_slots == ref.n_empty_slots
    assert info.kv_bytes == ref.kv_bytes
    assert info.merge_state_bytes == ref.merge_state_bytes
    assert info.n_buckets == len(ref.buckets)
    assert info.plan_bytes == got["total_words"] * 4
    assert info.max_task_pages == max((pe - pb for *_, pb, pe in ref.tasks), default=0)
    again = _lib.pkv_plan_get_info(prob, _plan_buf(prob, lens, path, s))
    assert again.as_dict() == info.as_dict()
    # The planner uses the buffer's tail as scratch: prior contents must not matter.
    dirty = np.full(_lib.pkv_plan_bytes(prob, path, s) // 4, -12345, dtype=np.int32)
    _lib.pkv_plan(prob, np.asarray(lens, dtype=np.int32), path, s, dirty)
    clean = _plan_buf(prob, lens, path, s)
    n = got["total_words"]
    np.testing.assert_array_equal(dirty[:n], clean[:n])


def _plan_buf(prob, lens, path, s):
    buf = np.zeros(_lib.pkv_plan_bytes(prob, path, s) // 4, dtype=np.int32)
    _lib.pkv_plan(prob, np.asarray(lens, dtype=np.int32), path, s, buf)
    return buf


def test_fanout_16_to_2_through_the_c_planner():
    rng = np.random.default_rng(20260623)
    lens = np.concatenate([rng.integers(128, 2048, 4, endpoint=True),
                           rng.integers(16384, 32768, 4, endpoint=True)])
    prob = _prob(8)
    assert _plan(prob, lens, PKV_BUCKETED, 32)[0].n_launches == 16
    assert _plan(prob, lens, PKV_WORKQUEUE, 32)[0].n_launches == 2


@pytest.mark.parametrize("seed", range(10))
def test_policy_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    rules = []
    for _ in range(int(rng.integers(1, 8))):
        b_lo = int(rng.integers(1, 40))
        n_lo = int(rng.integers(0, 20000))
        rules.append((b_lo, b_lo + int(rng.integers(0, 40)), n_lo, n_lo + int(rng.integers(0, 20000)),
                      int(rng.integers(0, 4)), int(rng.integers(1, 65))))
    for _ in range(200):
        b, n = int(rng.integers(1, 80)), int(rng.integers(0, 40000))
        ref = oracle_choose(rules, b, n)
        if ref is None:
            with pytest.raises(PkvError) as e:
                _lib.pkv_policy(rules, b, n)
            assert e.value.status == PKV_ERANGE
        else:
            assert _lib.pkv_policy(rules, b, n) == ref


def test_policy_errors():
    with pytest.raises(PkvError) as e:
        _lib.pkv_policy([(1, 1, 0, 10, 7, 1)], 1, 1)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_policy([(1, 1, 0, 10, 1, 0)], 1, 1)
    assert e.value.status == PKV_EINVAL


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 30, PKV_ESHAPE),   # Hq % Hkv != 0
    ("num_q_heads", 8 * 17, PKV_ESHAPE),  # G = 17 > 16
    ("head_dim", 96, PKV_ESHAPE),
    ("page_size", 8, PKV_ESHAPE),
    ("dtype", 7, PKV_EDTYPE),
    ("batch", 0, PKV_EINVAL),
    ("kernel", 9, PKV_EINVAL),
    ("num_pool_pages", 0, PKV_EINVAL),
    ("max_pages_per_row", 1 << 27, PKV_ESHAPE),  # token indices past 32 bits
])
def test_plan_rejects_bad_problems(field, value, status):
    prob = _prob(2)
    setattr(prob, field, value)
    buf = np.zeros(1 << 16, dtype=np.int32)
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan(prob, np.array([5, 6], np.int32), PKV_WORKQUEUE, 4, buf)
    assert e.value.status == status
    assert _lib.pkv_plan_bytes(prob, PKV_WORKQUEUE, 4) == 0


def test_plan_rejects_bad_lengths_splits_and_small_buffers():
    prob = _prob(2, max_pages=4)
    buf = np.zeros(1 << 12, dtype=np.int32)
    for lens in ([65, 1], [-1, 3]):
        with pytest.raises(PkvError) as e:
            _lib.pkv_plan(prob, np.array(lens, np.int32), PKV_WORKQUEUE, 4, buf)
        assert e.value.status == PKV_ERANGE
    _lib.pkv_plan(prob, np.array([64, 0], np.int32), PKV_WORKQUEUE, 4, buf)  # at capacity
    for s in (0, 70000):
        with pytest.raises(PkvError) as e:
            _lib.pkv_plan(prob, np.array([5, 1], np.int32), PKV_WORKQUEUE, s, buf)
        assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan(prob, np.array([5, 1], np.int32), 4, 4, buf)
    assert e.value.status == PKV_EINVAL
    need = _lib.pkv_plan_bytes(prob, PKV_WORKQUEUE, 4)
    small = np.zeros(need // 4 - 1, dtype=np.int32)
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan(prob, np.array([5, 1], np.int32), PKV_WORKQUEUE, 4, small,
                      plan_bytes=small.nbytes)
    assert e.value.status == PKV_ENOSPC


def test_decode_and_merge_validate_before_launch():
    prob = _prob(2)
    buf = _plan_buf(prob, [40, 3], PKV_WORKQUEUE, 4)
    other = _prob(3)
    fake = 0x1000  # never dereferenced: every call below fails validation first
    with pytest.raises(PkvError) as e:  # plan made for another batch size
        _lib.pkv_decode(other, buf, fake, fake, fake, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ESHAPE
    with pytest.raises(PkvError) as e:  # missing q
        _lib.pkv_decode(prob, buf, fake, None, fake, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:  # missing states on a split path
        _lib.pkv_decode(prob, buf, fake, fake, fake, fake, fake, fake, None, None, None)
    assert e.value.status == PKV_EINVAL
    # Kernel / shape combinations no split kernel covers, caught before launch.
    for hq, hkv, d, kernel in ((32, 2, 64, _lib.PKV_KERNEL_AUTO),    # d=64 needs G <= 8
                               (32, 2, 128, _lib.PKV_KERNEL_VALU),   # VALU: G <= 8
                               (8, 2, 64, _lib.PKV_KERNEL_MFMA)):    # MFMA: d = 128 only
        pr = _prob(2, hq=hq, hkv=hkv, d=d)
        pr.kernel = kernel
        pb = _plan_buf(pr, [40, 3], PKV_WORKQUEUE, 4)
        with pytest.raises(PkvError) as e:
            _lib.pkv_decode(pr, pb, fake, fake, fake, fake, fake, fake, fake, fake, fake)
        assert e.value.status == PKV_ESHAPE, (hq, hkv, d, kernel)
    bad = buf.copy()
    bad[0] = 0
    with pytest.raises(PkvError) as e:  # not a plan
        _lib.pkv_merge(prob, bad, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:  # missing output
        _lib.pkv_merge(prob, buf, fake, fake, fake, fake, None)
    assert e.value.status == PKV_EINVAL
    bad_dt = _prob(2, dtype="f16")
    bad_dt.dtype = 5
    with pytest.raises(PkvError) as e:
        _lib.pkv_merge(bad_dt, buf, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_EDTYPE


def test_launches_past_the_dispatch_limit_are_rejected_before_launch():
    """A launch's work-item count (workgroups x threads) must fit 32 bits; the
    library rejects grids of more than 2^24 - 1 workgroups with ERANGE before
    enqueuing anything.  Lengths are zero or one page, so the plans touch
    little memory (np.zeros pages are allocated lazily)."""
    fake = 0x1000  # never dereferenced: every call below fails validation first
    limit = (1 << 24) - 1
    # Merge: B x Hq workgroups.
    prob = _prob(65536, hq=256, hkv=16, max_pages=4)
    assert 65536 * 256 > limit
    buf = _plan_buf(prob, np.zeros(65536, np.int32), PKV_WORKQUEUE, 1)
    with pytest.raises(PkvError) as e:
        _lib.pkv_merge(prob, buf, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ERANGE
    # No-split decode: B x Hkv workgroups; append: the same grid.
    prob = _prob(1 << 20, hq=16, hkv=16, max_pages=4)
    buf = _plan_buf(prob, np.zeros(1 << 20, np.int32), PKV_NOSPLIT, 1)
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode(prob, buf, fake, fake, fake, fake, fake, fake, None, None, None, fake)
    assert e.value.status == PKV_ERANGE
    with pytest.raises(PkvError) as e:
        _lib.pkv_append_kv(prob, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ERANGE
    # Bucketed decode: rows_b x Hkv x S slots in one bucket's launch.
    prob = _prob(32, hq=16, hkv=16, max_pages=4)
    assert 32 * 16 * 65535 > limit
    buf = _plan_buf(prob, np.full(32, 16, np.int32), PKV_BUCKETED, 65535)
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode(prob, buf, fake, fake, fake, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ERANGE
    # Bucketed decode: a bucket's rows are its launch's third grid dimension,
    # at most 65535, even when the slot count is far below the limit.
    prob = _prob(65536, hq=1, hkv=1, max_pages=4)
    buf = _plan_buf(prob, np.full(65536, 16, np.int32), PKV_BUCKETED, 1)
    assert 65536 * 1 * 1 <= limit
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode(prob, buf, fake, fake, fake, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ERANGE


def test_status_strings():
    for s in range(-6, 1):
        assert _lib.pkv_status_str(s)
    assert _lib.pkv_status_str(-99) == "unknown status"


def test_device_plan_entry_points_validate_before_launch():
    prob = _prob(2)
    fake = 0x1000  # never dereferenced: every call below fails validation first
    need = _lib.pkv_plan_bytes(prob, PKV_WORKQUEUE, 8)
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan_device(prob, None, 8, fake, need)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan_device(prob, fake, 8, fake, need - 4)
    assert e.value.status == PKV_ENOSPC
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan_device(prob, fake, 0, fake, need)
    assert e.value.status == PKV_EINVAL
    big = _prob(16385)  # one row past the device planner's limit
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan_device(big, fake, 8, fake, _lib.pkv_plan_bytes(big, PKV_WORKQUEUE, 8))
    assert e.value.status == PKV_ERANGE
    wide = _prob(16384, hq=4096, hkv=4096)  # a plan of more than 2^31 - 1 words
    need = _lib.pkv_plan_bytes(wide, PKV_WORKQUEUE, 64)
    assert need // 4 > 2**31 - 1
    with pytest.raises(PkvError) as e:
        _lib.pkv_plan_device(wide, fake, 64, fake, need)
    assert e.value.status == PKV_ERANGE
    # Shapes no split kernel covers: d = 64 needs the vector-ALU kernel, which
    # takes G <= 8; so does an explicit vector-ALU request.
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode_device(_prob(2, hq=32, hkv=2, d=64), fake, 8, fake, fake, fake, fake, fake,
                               fake, fake)
    assert e.value.status == PKV_ESHAPE
    valu = _prob(2, hq=32, hkv=2)
    valu.kernel = _lib.PKV_KERNEL_VALU
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode_device(valu, fake, 8, fake, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ESHAPE
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode_device(prob, fake, 8, fake, None, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_merge_device(prob, fake, fake, fake, fake, None)
    assert e.value.status == PKV_EINVAL


def test_selfplan_entry_points_validate_before_launch():
    prob = _prob(2)
    fake = 0x1000  # never dereferenced: every call below fails validation first
    args = (fake, fake, fake, fake, fake, fake, fake)  # q, k, v, table, st_m, st_l, st_o
    with pytest.raises(PkvError) as e:  # no claim counter
        _lib.pkv_decode_selfplan(prob, fake, 8, None, *args)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode_selfplan(prob, fake, 0, fake, *args)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:  # one row past the in-kernel planning limit
        _lib.pkv_decode_selfplan(_prob(1025), fake, 8, fake, *args)
    assert e.value.status == PKV_ERANGE
    with pytest.raises(PkvError) as e:  # B * Hkv * S past 32-bit task indices
        _lib.pkv_decode_selfplan(_prob(1024, hq=4096, hkv=4096), fake, 65535, fake, *args)
    assert e.value.status == PKV_ERANGE
    with pytest.raises(PkvError) as e:  # d = 64 with G = 16: no split kernel covers it
        _lib.pkv_decode_selfplan(_prob(2, hq=32, hkv=2, d=64), fake, 8, fake, *args)
    assert e.value.status == PKV_ESHAPE
    valu = _prob(2, hq=32, hkv=2)  # the vector-ALU kernel takes G <= 8
    valu.kernel = _lib.PKV_KERNEL_VALU
    with pytest.raises(PkvError) as e:
        _lib.pkv_decode_selfplan(valu, fake, 8, fake, *args)
    assert e.value.status == PKV_ESHAPE
    with pytest.raises(PkvError) as e:  # missing states
        _lib.pkv_decode_selfplan(prob, fake, 8, fake, fake, fake, fake, fake, None, fake, fake)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:  # missing output
        _lib.pkv_merge_selfplan(prob, fake, 8, fake, fake, fake, fake, None)
    assert e.value.status == PKV_EINVAL
    with pytest.raises(PkvError) as e:
        _lib.pkv_merge_selfplan(_prob(1025), fake, 8, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ERANGE


def test_append_validates_before_launch():
    prob = _prob(2)
    fake = 0x1000
    with pytest.raises(PkvError) as e:
        _lib.pkv_append_kv(prob, fake, None, fake, fake, fake, fake)
    assert e.value.status == PKV_EINVAL
    bad = _prob(2)
    bad.head_dim = 96
    with pytest.raises(PkvError) as e:
        _lib.pkv_append_kv(bad, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ESHAPE


def test_probe_library_exports_its_header():
    from paged_kv_gqa_block_amd import probe

    with open(os.path.join(os.path.dirname(HEADER), "pkv_probe.h")) as f:
        declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(pkv_\w+)\s*\(", f.read(), flags=re.M))
    assert declared == set(probe.EXPORTED)
    for name in declared:
        assert hasattr(probe.LIB, name), name


def test_noalloc_scratch_size_and_limit():
    """pkv_noalloc_bytes is the closed form (three 256-byte aligned arrays of
    B * Hkv * S slots: m and l of G floats, o of G * d floats); a call needing
    more than the library's array fails with PKV_ENOSPC before any GPU work."""
    prob = _prob(8, hq=32, hkv=8, d=128)
    slots, g = 8 * 8 * 32, 4

    def r256(n):
        return (n + 255) // 256 * 256

    assert _lib.pkv_noalloc_bytes(prob, 32) == 2 * r256(slots * g * 4) + r256(slots * g * 128 * 4)
    assert _lib.pkv_noalloc_bytes(prob, 0) == 0
    big = _prob(1024, hq=64, hkv=8, d=128)
    assert _lib.pkv_noalloc_bytes(big, 64) > _lib.PKV_NOALLOC_SCRATCH_BYTES
    fake = 4096
    with pytest.raises(PkvError) as e:
        _lib.pkv_attend_noalloc(big, fake, 64, fake, fake, fake, fake, fake, fake)
    assert e.value.status == PKV_ENOSPC
    with pytest.raises(PkvError) as e:
        _lib.pkv_attend_noalloc(prob, fake, 32, fake, fake, fake, fake, None, fake)
    assert e.value.status == PKV_EINVAL
