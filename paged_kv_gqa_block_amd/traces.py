"""Seeded synthetic decode workloads for paged grouped-query attention.

This module only draws numbers: per-row context lengths, a shuffled page pool,
and the q / K / V values. It holds none of the attention, planning or merge
arithmetic, so the CPU oracle and the HIP path can both be fed from it without
sharing any of the method's code.

Workload shapes follow the PersistentKV summary pages ("PersistentKV:
Page-Aware Decode Scheduling for Long-Context LLM Serving on Commodity GPUs",
section "Evaluation Protocol": synthetic Bucketed / Bimodal / Uniform / Zipf
traces chosen to isolate context length, active batch size and length
irregularity; section "Results": calibration seed 20260622, held-out seed
20260623). The concrete sizes (heads, head_dim, page size, length ranges) are
this project's choice; the pages give none.

Draw order for one workload, from ``numpy.random.default_rng(seed)``:
lengths, then the pool permutation, then q, then the K pool, then the V pool.
Values are standard normal float32 rounded to nearest-even into fp16 or bf16.
Block tables take the first sum(T_i) entries of the permutation, cut
consecutively by row, so no two rows share a page.  With ``poison=True`` every
pool page that no row uses, and every slot past a row's last real token in its
last page, is set to NaN; block-table entries past a row's last page point at
an unused (NaN) page when one exists.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

CALIBRATION_SEED = 20260622
HELD_OUT_SEED = 20260623
POLICY_BATCHES = (1, 2, 4, 8, 16, 32, 64)

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape of one synthetic decode step (one layer)."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    lengths: str  # "fixed" | "bimodal" | "zipf" | "uniform"
    splits: int
    dtype: str = "f16"
    fixed_len: int = 0
    lo: int = 0
    hi: int = 0
    pool_pages: Optional[int] = None  # None: ceil(1.5 * sum(T_i))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _spec_table():
    specs = {
        # B=1, 8/2 heads, d=64, N=2048, 256-page pool, S=4.
        "tiny": WorkloadSpec("tiny", 1, 8, 2, 64, 16, "fixed", 4, "f16", fixed_len=2048,
                             pool_pages=256),
        # B=1, 32/8 heads, d=128, N=32768, pool 1.5x the pages needed, S=32.
        "long": WorkloadSpec("long", 1, 32, 8, 128, 16, "fixed", 32, "f16", fixed_len=32768),
        # B=8, half U[128,2048] and half U[16384,32768], up to 32 splits per row.
        "bimodal": WorkloadSpec("bimodal", 8, 32, 8, 128, 16, "bimodal", 32, "f16"),
        # B=8, clip(64 * Zipf(1.2), 64, 32768).
        "zipf": WorkloadSpec("zipf", 8, 32, 8, 128, 16, "zipf", 32, "f16", lo=64, hi=32768),
        # B=8, U[1024,32768] with the long-context head shape (fourth trace family).
        "uniform": WorkloadSpec("uniform", 8, 32, 8, 128, 16, "uniform", 32, "f16",
                                lo=1024, hi=32768),
    }
    for b in POLICY_BATCHES:
        # Policy sweep: 64/8 heads, d=128, bf16, U[1024,32768].
        specs[f"policy_b{b}"] = WorkloadSpec(f"policy_b{b}", b, 64, 8, 128, 16, "uniform", 32,
                                             "bf16", lo=1024, hi=32768)
        # Short-context band of the same shape, U[64,2048], so the calibrated
        # table also has an N_max split.
        specs[f"policy_short_b{b}"] = WorkloadSpec(f"policy_short_b{b}", b, 64, 8, 128, 16,
                                                   "uniform", 32, "bf16", lo=64, hi=2048)
    return specs


SPECS = _spec_table()


def get_spec(name: str, **overrides) -> WorkloadSpec:
    spec = SPECS[name]
    return dataclasses.replace(spec, **overrides) if overrides else spec


def draw_lengths(spec: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    b = spec.batch
    if spec.lengths == "fixed":
        lens = np.full(b, spec.fixed_len, dtype=np.int64)
    elif spec.lengths == "bimodal":
        short = rng.integers(128, 2048, size=b // 2, endpoint=True)
        long = rng.integers(16384, 32768, size=b - b // 2, endpoint=True)
        lens = np.concatenate([short, long])
        rng.shuffle(lens)
    elif spec.lengths == "zipf":
        k = rng.zipf(1.2, size=b)
        lens = np.clip(64 * k.astype(np.float64), spec.lo, spec.hi).astype(np.int64)
    elif spec.lengths == "uniform":
        lens = rng.integers(spec.lo, spec.hi, size=b, endpoint=True)
    else:
        raise ValueError(f"unknown length distribution {spec.lengths!r}")
    return lens.astype(np.int32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    # torch's CPU float32 -> fp16/bf16 conversion rounds to nearest-even.
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def generate(spec: WorkloadSpec, seed: int, poison: bool = True,
             seq_lens: Optional[np.ndarray] = None) -> dict:
    """Draw one decode step.  Returns CPU tensors and the problem sizes.

    ``seq_lens`` (optional) replaces the drawn lengths; the length draw still
    happens first so the rest of the stream stays aligned with the spec.
    """
    rng = np.random.default_rng(seed)
    lens = draw_lengths(spec, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (spec.batch,)
    p = spec.page_size
    pages_per_row = [(int(n) + p - 1) // p for n in lens]
    used = int(sum(pages_per_row))
    pool = spec.pool_pages if spec.pool_pages is not None else (3 * used + 1) // 2
    pool = max(pool, used, 1)
    perm = rng.permutation(pool).astype(np.int32)

    q = _normal(rng, (spec.batch, spec.num_q_heads, spec.head_dim), spec.dtype)
    pool_shape = (pool, spec.num_kv_heads, p, spec.head_dim)
    k_pool = _normal(rng, pool_shape, spec.dtype)
    v_pool = _normal(rng, pool_shape, spec.dtype)

    max_pages = max(1, max(pages_per_row) if pages_per_row else 1)
    unused = perm[used:]
    filler = int(unused[0]) if (poison and unused.size) else 0
    block_table = np.full((spec.batch, max_pages), filler, dtype=np.int32)
    off = 0
    for i, t in enumerate(pages_per_row):
        block_table[i, :t] = perm[off:off + t]
        off += t

    if poison:
        nan = float("nan")
        if unused.size:
            idx = torch.from_numpy(unused.astype(np.int64))
            k_pool[idx] = nan
            v_pool[idx] = nan
        for i, n in enumerate(lens):
            t = pages_per_row[i]
            tail = int(n) - (t - 1) * p
            if t and tail < p:
                last = int(block_table[i, t - 1])
                k_pool[last, :, tail:, :] = nan
                v_pool[last, :, tail:, :] = nan

    scale = float(np.float32(1.0 / np.sqrt(spec.head_dim)))
    return {
        "spec": spec,
        "seed": seed,
        "q": q,
        "k_pool": k_pool,
        "v_pool": v_pool,
        "block_table": torch.from_numpy(block_table),
        "seq_lens": torch.from_numpy(lens.copy()),
        "scale": scale,
        "num_pool_pages": pool,
    }


def custom_spec(batch, num_q_heads, num_kv_heads, head_dim, page_size=16, splits=4,
                dtype="f16", pool_pages=None, name="custom") -> WorkloadSpec:
    """A spec whose lengths are always supplied through ``generate(seq_lens=...)``."""
    return WorkloadSpec(name, batch, num_q_heads, num_kv_heads, head_dim, page_size, "fixed",
                        splits, dtype, fixed_len=0, pool_pages=pool_pages)


def oracle_arrays(w: dict) -> dict:
    """The same tensors as numpy arrays in their stored encoding.

    fp16 stays ``numpy.float16``; bf16 is handed over as its raw uint16 bit
    patterns (numpy has no bf16 type).
    """
    def enc(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return t.contiguous().numpy()

    return {
        "q": enc(w["q"]),
        "k_pool": enc(w["k_pool"]),
        "v_pool": enc(w["v_pool"]),
        "block_table": w["block_table"].numpy(),
        "seq_lens": w["seq_lens"].numpy(),
        "scale": w["scale"],
        "dtype": w["spec"].dtype,
        "page_size": w["spec"].page_size,
    }
