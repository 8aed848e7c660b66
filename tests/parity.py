"""Shared comparison rules for the GPU parity tests (not a test module).

Tolerances (reading of "FP16 tolerance", which the pages give without a
number; the bound is max-abs <= 2e-3 and relative L2 <= 1e-3):
* fp16 output vs the raw fp64 oracle.
* bf16 output vs the fp64 oracle rounded to bf16 (nearest-even), because the
  output rounding alone already exceeds 1e-3 relative L2 for bf16.  An
  element may also differ by one bf16 unit in the last place, which happens
  when the fp32 kernel result and the fp64 value straddle a rounding midpoint.
* lse (natural log) within 2e-4 absolute.
* partial states: lse_s = m + ln l within 2e-4, o/l within 1e-4 (max-abs).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_kv_gqa_block_amd import traces

MAX_ABS = 2e-3
REL_L2 = 1e-3
LSE_ABS = 2e-4


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def oracle_out(w: dict, rows=None):
    a = traces.oracle_arrays(w)
    return oracle.attention(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"],
                            a["scale"], a["page_size"], a["dtype"], rows=rows)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_out(got: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, label=""):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{label}: non-finite output"
    if dtype == "bf16":
        r = oracle.round_to_bf16(ref)
        diff = np.abs(g - r)
        allowed = np.maximum(MAX_ABS, bf16_ulp(r) * 1.0001)
        bad = diff > allowed
        assert not bad.any(), f"{label}: {bad.sum()} elements beyond max(2e-3, 1 ulp); " \
                              f"worst {diff.max():.3e}"
    else:
        r = ref
        diff = np.abs(g - r)
        assert diff.max() <= MAX_ABS, f"{label}: max-abs {diff.max():.3e}"
    denom = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / denom if denom > 0 else np.linalg.norm(g - r)
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e}"
    return float(diff.max()), float(rel)


def check_lse(got: torch.Tensor, ref: np.ndarray, rows=None, label=""):
    g = got.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{label}: -inf pattern differs"
    fin = np.isfinite(ref)
    if fin.any():
        err = np.abs(g[fin] - ref[fin]).max()
        assert err <= LSE_ABS, f"{label}: lse abs err {err:.3e}"
