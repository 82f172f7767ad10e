"""Oracle work of the full-size GPU parity tests, run in worker processes.

The Nside = 64 / 128 / 256 workloads hold 32 to 192 (batch, head) slices.
Checking every selected-block row of every slice, and every output element
of a set of whole slices, against the float64 oracle takes minutes on one
core, so the tests hand each slice to a pool of host processes.  A job gets
one slice's exact input bits (bf16 as uint16, gates float32) and the GPU's
results for it, runs the oracle and returns what it found; the parent
asserts.  This module imports numpy, the oracle and the comparison helpers
only: workers never touch the GPU.
"""

from __future__ import annotations

import multiprocessing
import os

import numpy as np

import oracle
from parity import check_indices, error_stats, selection_ref


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the same values as float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def index_job(tag, q_bits, k_bits, v_bits, block: int, topn: int, gpu_idx) -> dict:
    """Every index row of one slice against the oracle's pooling, compressed
    logits and top-n (bit-exact except near-tie rows, which must be top-n
    within the slack)."""
    q, k, v = widen_bf16(q_bits), widen_bf16(k_bits), widen_bf16(v_bits)
    ref = selection_ref(q, k, v, block, topn)
    try:
        st = check_indices(np.asarray(gpu_idx), ref, topn)
    except AssertionError as e:
        return dict(tag=tag, ok=False, msg=str(e))
    return dict(tag=tag, ok=True, rows=st["rows"], near_ties=st["near_ties"])


def output_job(tag, q_bits, k_bits, v_bits, gates, block: int, topn: int, window: int, gpu_idx, gpu_out) -> dict:
    """Every output element of one slice against the oracle run with the GPU's
    own selection (which index_job checks against the oracle's)."""
    q, k, v = widen_bf16(q_bits), widen_bf16(k_bits), widen_bf16(v_bits)
    ref = oracle.bsa_slice_ref(q, k, v, np.asarray(gates, dtype=np.float64), block, topn, window,
                               idx=np.asarray(gpu_idx))
    got = np.asarray(gpu_out, dtype=np.float64)
    max_abs, rel = error_stats(got, ref["out"])
    return dict(tag=tag, finite=bool(np.all(np.isfinite(got))), max_abs=max_abs, rel=rel,
                diff2=float(np.sum((got - ref["out"]) ** 2)), ref2=float(np.sum(ref["out"] ** 2)))


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def workers() -> int:
    """Host processes for the oracle: the CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def pool():
    """A multiprocessing pool of fresh interpreters (spawned: nothing of the
    parent's GPU state is inherited) with one BLAS thread each.  The workers
    start inside this call, with the thread variables set to 1 for them
    only."""
    saved = {var: os.environ.get(var) for var in _THREAD_VARS}
    os.environ.update({var: "1" for var in _THREAD_VARS})
    try:
        return multiprocessing.get_context("spawn").Pool(workers(), initializer=_one_thread)
    finally:
        for var, val in saved.items():
            if val is None:
                os.environ.pop(var, None)
            else:
                os.environ[var] = val
