"""Comparison helpers shared by the GPU parity tests (HIP path vs float64 oracle).

Tolerances (fixed by the workload definition for bf16 inputs with float32
accumulation): max-abs 1e-2 and relative L2 5e-3 on the output; selected
block indices bit-exact on every row whose n-th and (n+1)-th compressed
logits differ by 1e-6 or more (or are exactly equal, where the lower-index
rule decides); rows with 0 < gap < 1e-6 are near-ties, where any top-n set
within 1e-6 of optimal is accepted and outputs are compared against the
oracle run with the GPU's own indices.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle

MAX_ABS = 1e-2
REL_L2 = 5e-3
NEAR_TIE = 1e-6


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def selection_ref(q, k, v, block, topn):
    """Oracle pooled tensors, logits, indices and gaps of one slice."""
    qbar, kbar, vbar = oracle.pool_mean(q, block), oracle.pool_mean(k, block), oracle.pool_mean(v, block)
    s, _, o_cg = oracle.compressed_branch(qbar, kbar, vbar)
    idx, gap = oracle.select_topn(s, topn)
    return dict(qbar=qbar, kbar=kbar, vbar=vbar, s=s, o_cg=o_cg, idx=idx, gap=gap)


def ocg_tolerance(vbar: np.ndarray) -> float:
    """Bound on |o_CG(gpu) - o_CG(oracle)| elementwise.  The kernel rounds the
    softmax weights and v̄ to bf16 (relative error <= 2^-9 each) and sums the
    rounded weights for the denominator: the normalised weights then err by
    at most 2 * 2^-9 relative and sum to one, so o_CG errs by at most
    (2 + 1) * 2^-9 * max|v̄|, plus float32 accumulation."""
    return 3.0 * 2.0 ** -9 * float(np.abs(vbar).max()) + 2e-5


def check_indices(gpu_idx: np.ndarray, ref: dict, topn: int) -> dict:
    """Bit-exact on non-near-tie rows; top-n-within-slack on near-tie rows."""
    idx, gap, s = ref["idx"], ref["gap"], ref["s"]
    m = s.shape[1]
    near = (gap > 0) & (gap < NEAR_TIE)
    exact = ~near
    bad = np.nonzero(np.any(gpu_idx[exact] != idx[exact], axis=1))[0]
    assert bad.size == 0, (f"{bad.size} index rows differ, first row {np.nonzero(exact)[0][bad[0]]}: "
                           f"gpu {gpu_idx[exact][bad[0]]} vs oracle {idx[exact][bad[0]]}")
    for r in np.nonzero(near)[0]:
        sel = gpu_idx[r]
        assert np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() < m
        rest = np.setdiff1d(np.arange(m), sel)
        if rest.size:
            assert s[r, sel].min() >= s[r, rest].max() - NEAR_TIE
    return dict(rows=int(gap.size), near_ties=int(near.sum()))


def error_stats(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return max_abs, rel


def assert_close(got, want, what: str, max_abs: float = MAX_ABS, rel_l2: float = REL_L2):
    a, r = error_stats(got, want)
    log(f"    {what}: max-abs {a:.3e}  rel-L2 {r:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert a <= max_abs, f"{what}: max-abs {a:.3e} > {max_abs}"
    assert r <= rel_l2, f"{what}: rel-L2 {r:.3e} > {rel_l2}"
    return a, r
