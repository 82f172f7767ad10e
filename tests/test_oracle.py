"""Pins of the float64 BSA oracle against things other than itself.

Each pin is a closed form, a special case that reduces to a library routine
(torch's float64 scaled_dot_product_attention, computed on the CPU), a brute
force written independently of the oracle's vectorised code, or an invariant.
The definition being pinned: papernotes.org ICML2026 notes, 关键设计 ›
Mesh-aligned Block-Sparse Attention (BSA).

Plausible mistakes and the pins that catch them:
  missing / wrong 1/sqrt(d) scale ............ sdpa pins (every branch)
  transposed q/k or v operand ................ sdpa pins
  per-block instead of union softmax (FG) .... test_fine_all_blocks_is_dense
  wrong selection direction / tie-break ...... brute-force order, hand example, q̄ = 0
  off-centre or causal window ................ band-mask sdpa pin, W = 1, q = 0 means
  wrong gate column / block broadcast ........ one-hot gates, B = 1 whole-op pin
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bsa

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def sdpa(q, k, v, mask=None):
    """Library routine: torch float64 scaled-dot-product attention on the CPU."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    with torch.no_grad():
        return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)[0].numpy()


def dense_bruteforce(q, k, v):
    """Naive dense softmax attention, one query at a time in plain Python
    floats (math.exp / math.fsum), written apart from the oracle's numpy code."""
    n, d = q.shape
    out = np.zeros((n, v.shape[1]))
    for t in range(n):
        s = [math.fsum(q[t, c] * k[u, c] for c in range(d)) / math.sqrt(d) for u in range(k.shape[0])]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = math.fsum(w)
        for c in range(v.shape[1]):
            out[t, c] = math.fsum(w[u] * v[u, c] for u in range(k.shape[0])) / z
    return out


# ---------------------------------------------------------------- pooling ---

def test_pool_block_constant():
    B, m, d = 16, 12, 8
    const = _rand(m, d)
    x = np.repeat(const, B, axis=0)
    np.testing.assert_allclose(oracle.pool_mean(x, B), const, rtol=1e-15, atol=0)
    # with values whose sums are exact (bf16-representable), the mean is exact
    c16 = np.round(const * 64) / 64
    np.testing.assert_array_equal(oracle.pool_mean(np.repeat(c16, B, axis=0), B), c16)


def test_pool_linear_ramp_closed_form():
    # x_t = a*t + c  ->  mean over block i = a*(i*B + (B-1)/2) + c
    B, m = 64, 48
    a, c = 0.25, -3.0
    t = np.arange(m * B, dtype=np.float64)
    x = np.stack([a * t + c, -2 * a * t], axis=1)
    i = np.arange(m)
    want = np.stack([a * (i * B + (B - 1) / 2) + c, -2 * a * (i * B + (B - 1) / 2)], axis=1)
    np.testing.assert_allclose(oracle.pool_mean(x, B), want, rtol=0, atol=1e-12)


def test_pool_exact_on_bf16_values():
    # block means of bf16-valued data are exact in float64 (B is a power of two)
    B = 256
    x = torch.randn(12 * B, 4, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    xd = x.double().numpy()
    want = np.array([[math.fsum(xd[i * B:(i + 1) * B, c]) / B for c in range(4)] for i in range(12)])
    np.testing.assert_array_equal(oracle.pool_mean(xd, B), want)


# -------------------------------------------------------- compressed branch ---

def test_compressed_block1_is_dense_attention():
    n, d = 192, 16
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    _, _, o_cg = oracle.compressed_branch(q, k, v)       # B = 1: q̄ = q, ...
    np.testing.assert_allclose(o_cg, sdpa(q, k, v), rtol=0, atol=1e-12)


def test_compressed_zero_query_is_global_mean():
    n, B, d = 768, 16, 32
    k, v = _rand(n, d), _rand(n, d)
    q = np.zeros((n, d))
    r = oracle.bsa_slice_ref(q, k, v, np.ones((n, 3)), B, 4, 32)
    np.testing.assert_allclose(r["o_cg"], np.broadcast_to(v.mean(axis=0), r["o_cg"].shape), atol=1e-13)


def test_compressed_scores_scale_and_softmax():
    m, d = 48, 32
    qb, kb, vb = _rand(m, d), _rand(m, d), _rand(m, d)
    s, a, o = oracle.compressed_branch(qb, kb, vb)
    # attention weights from the library (values = identity) equal the softmax of s
    np.testing.assert_allclose(a, sdpa(qb, kb, np.eye(m)), atol=1e-13)
    # and a few logits by brute force
    for i, j in [(0, 0), (3, 17), (47, 46)]:
        assert abs(s[i, j] - math.fsum(qb[i] * kb[j]) / math.sqrt(d)) < 1e-13
    np.testing.assert_allclose(a.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(o, sdpa(qb, kb, vb), atol=1e-12)


# ---------------------------------------------------------------- selection ---

def test_select_hand_example_ties():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0],
                  [-1.0, 5.0, -2.0, 5.0, 4.0]])
    idx, gap = oracle.select_topn(s, 2)
    np.testing.assert_array_equal(idx, [[1, 2], [0, 1], [1, 3]])
    np.testing.assert_array_equal(gap, [0.0, 0.0, 1.0])
    idx3, gap3 = oracle.select_topn(s, 3)
    np.testing.assert_array_equal(idx3, [[1, 2, 4], [0, 1, 2], [1, 3, 4]])
    np.testing.assert_array_equal(gap3, [1.0, 0.0, 5.0])


def test_select_bruteforce_definition():
    """Every selected j beats every unselected u under (larger logit, then
    lower index); checked pair by pair in plain Python."""
    m, n = 48, 4
    s = np.round(_rand(40, m), 1)          # rounding makes many exact ties
    idx, gap = oracle.select_topn(s, n)
    for r in range(s.shape[0]):
        sel = list(idx[r])
        assert sel == sorted(sel) and len(set(sel)) == n
        for j in sel:
            for u in range(m):
                if u in sel:
                    continue
                assert s[r, j] > s[r, u] or (s[r, j] == s[r, u] and j < u)
        ordered = sorted(range(m), key=lambda u: (-s[r, u], u))
        assert gap[r] == s[r, ordered[n - 1]] - s[r, ordered[n]]


def test_select_zero_logits_and_all():
    s = np.zeros((5, 48))
    idx, _ = oracle.select_topn(s, 7)
    np.testing.assert_array_equal(idx, np.tile(np.arange(7), (5, 1)))
    idx, gap = oracle.select_topn(_rand(5, 48), 48)
    np.testing.assert_array_equal(idx, np.tile(np.arange(48), (5, 1)))
    assert np.all(np.isinf(gap))


def test_select_zero_block_mean_query():
    # q alternating in sign inside each block -> q̄ = 0 -> all logits exactly 0
    n, B, d = 768, 16, 32
    q = np.repeat(_rand(n // 2, d), 2, axis=0) * np.tile([[1.0], [-1.0]], (n // 2, 1))
    r = oracle.bsa_slice_ref(q, _rand(n, d), _rand(n, d), np.ones((n, 3)), B, 4, 32)
    assert np.all(r["s"] == 0.0)
    np.testing.assert_array_equal(r["idx"], np.tile(np.arange(4), (n // B, 1)))


# --------------------------------------------------------- selected branch ---

def test_fine_all_blocks_is_dense():
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    m = n // B
    r = oracle.bsa_slice_ref(q, k, v, np.ones((n, 3)), B, m, 32)
    np.testing.assert_array_equal(r["idx"], np.tile(np.arange(m), (m, 1)))
    np.testing.assert_allclose(r["o_fg"], sdpa(q, k, v), rtol=0, atol=1e-12)


def test_fine_matches_library_block_mask():
    n, B, d, topn = 768, 16, 32, 5
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    m = n // B
    idx = np.sort(np.stack([RNG.choice(m, topn, replace=False) for _ in range(m)]), axis=1)
    o = oracle.fine_selected_branch(q, k, v, idx, B)
    sel = np.zeros((m, m), bool)
    sel[np.arange(m)[:, None], idx] = True
    mask = sel[np.arange(n)[:, None] // B, np.arange(n)[None, :] // B]
    np.testing.assert_allclose(o, sdpa(q, k, v, mask), rtol=0, atol=1e-12)


def test_fine_zero_query_closed_form():
    n, B, d = 768, 16, 32
    k, v = _rand(n, d), _rand(n, d)
    r = oracle.bsa_slice_ref(np.zeros((n, d)), k, v, np.ones((n, 3)), B, 4, 32)
    want = v[:4 * B].mean(axis=0)          # ties -> blocks 0..3, uniform weights
    np.testing.assert_allclose(r["o_fg"], np.broadcast_to(want, (n, d)), atol=1e-13)


def test_fine_invariant_to_permutation_inside_key_blocks():
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    perm = np.concatenate([i * B + RNG.permutation(B) for i in range(n // B)])
    a = oracle.bsa_slice_ref(q, k, v, np.ones((n, 3)), B, 4, 32)
    b = oracle.bsa_slice_ref(q, k[perm], v[perm], np.ones((n, 3)), B, 4, 32)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(a["o_fg"], b["o_fg"], atol=1e-13)


# ------------------------------------------------------------ local branch ---

@pytest.mark.parametrize("window", [1, 2, 7, 32, 33, 100])
def test_local_matches_library_band_mask(window):
    n, d = 192, 16
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    off = np.arange(n)[None, :] - np.arange(n)[:, None]       # u - t
    mask = (off >= -(window // 2)) & (off <= (window - 1) - window // 2)
    np.testing.assert_allclose(oracle.local_branch(q, k, v, window), sdpa(q, k, v, mask),
                               rtol=0, atol=1e-12)


def test_local_window_one_is_identity():
    n, d = 768, 32
    v = _rand(n, d)
    np.testing.assert_array_equal(oracle.local_branch(_rand(n, d), _rand(n, d), v, 1), v)


def test_local_huge_window_is_dense():
    n, d = 192, 16
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    np.testing.assert_allclose(oracle.local_branch(q, k, v, 2 * n), sdpa(q, k, v), atol=1e-12)


@pytest.mark.parametrize("window", [1, 4, 31, 32, 512])
def test_local_zero_query_clipped_window_means(window):
    n, d = 768, 8
    v = _rand(n, d)
    o = oracle.local_branch(np.zeros((n, d)), _rand(n, d), v, window)
    for t in [0, 1, 15, 16, 300, n - 17, n - 2, n - 1]:
        lo, hi = max(0, t - window // 2), min(n, t + (window + 1) // 2)
        assert hi - lo == min(n, t + (window + 1) // 2) - max(0, t - window // 2)
        np.testing.assert_allclose(o[t], v[lo:hi].mean(axis=0), atol=1e-13)
    # interior queries see exactly W keys
    lo, hi = oracle.local_window_bounds(np.arange(window, n - window), window, n)
    assert np.all(hi - lo == window)


# ------------------------------------------------------------ combination ---

def test_one_hot_gates_isolate_branches():
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    base = oracle.bsa_slice_ref(q, k, v, np.ones((n, 3)), B, 4, 32)
    for col, want in [(0, base["o_cg"][np.arange(n) // B]), (1, base["o_fg"]), (2, base["o_l"])]:
        g = np.zeros((n, 3))
        g[:, col] = 1.0
        r = oracle.bsa_slice_ref(q, k, v, g, B, 4, 32)
        np.testing.assert_array_equal(r["out"], want)
    np.testing.assert_allclose(base["out"], base["o_cg"][np.arange(n) // B] + base["o_fg"] + base["o_l"],
                               atol=1e-13)


def test_whole_op_degenerates_to_dense_bruteforce():
    """B = 1, n = m, W >= 2N: all three branches are dense attention, so
    out = (g0 + g1 + g2) * dense -- checked against a plain-Python brute force."""
    n, d = 48, 8                                        # Nside = 2
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    g = RNG.uniform(0, 1, (n, 3))
    r = oracle.bsa_slice_ref(q, k, v, g, 1, n, 2 * n)
    dense = dense_bruteforce(q, k, v)
    np.testing.assert_allclose(r["out"], g.sum(axis=1, keepdims=True) * dense, rtol=0, atol=1e-12)


def test_tiny_config_shapes_against_bruteforce_branches():
    """At the tiny workload's shape (N = 768, d = 32): with n = m the selected
    branch, and with W = 2N the local branch, equal the brute force."""
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    rows = np.array([0, 1, 100, 383, 767])
    dense = np.stack([_dense_row(q[t], k, v) for t in rows])
    r = oracle.bsa_slice_ref(q, k, v, np.ones((n, 3)), B, n // B, 2 * n)
    np.testing.assert_allclose(r["o_fg"][rows], dense, atol=1e-12)
    np.testing.assert_allclose(r["o_l"][rows], dense, atol=1e-12)


def _dense_row(qt, k, v):
    s = [math.fsum(qt * k[u]) / math.sqrt(qt.size) for u in range(k.shape[0])]
    mx = max(s)
    w = np.array([math.exp(x - mx) for x in s])
    return (w[:, None] * v).sum(axis=0) / math.fsum(w)


# --------------------------------------------------------- API consistency ---

def test_rows_variant_matches_slice():
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    g = RNG.uniform(0, 1, (n, 3))
    full = oracle.bsa_slice_ref(q, k, v, g, B, 4, 32)
    toks = np.array([0, 5, 16, 200, 767])
    rows = oracle.bsa_rows_ref(q, k, v, g, B, 4, 32, toks)
    np.testing.assert_allclose(rows["out"], full["out"][toks], atol=1e-13)
    for bk, sel in rows["idx"].items():
        np.testing.assert_array_equal(sel, full["idx"][bk])
        assert abs(rows["gap"][bk] - full["gap"][bk]) < 1e-12


def test_forced_indices():
    n, B, d = 768, 16, 32
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    g = RNG.uniform(0, 1, (n, 3))
    own = oracle.bsa_slice_ref(q, k, v, g, B, 4, 32)
    forced = oracle.bsa_slice_ref(q, k, v, g, B, 4, 32, idx=own["idx"])
    np.testing.assert_array_equal(own["out"], forced["out"])
    other = np.tile(np.arange(4), (n // B, 1))
    f2 = oracle.bsa_slice_ref(q, k, v, g, B, 4, 32, idx=other)
    np.testing.assert_allclose(f2["o_fg"], oracle.fine_selected_branch(q, k, v, other, B), atol=0)


def test_batched_wrapper():
    b, h, n, d, B = 1, 2, 768, 32, 16
    q, k, v = _rand(b, h, n, d), _rand(b, h, n, d), _rand(b, h, n, d)
    g = RNG.uniform(0, 1, (b, h, n, 3))
    r = oracle.bsa_forward_ref(q, k, v, g, B, 4, 32)
    for hi in range(h):
        s = oracle.bsa_slice_ref(q[0, hi], k[0, hi], v[0, hi], g[0, hi], B, 4, 32)
        np.testing.assert_array_equal(r["out"][0, hi], s["out"])
        np.testing.assert_array_equal(r["idx"][0, hi], s["idx"])


def test_shape_validation():
    q = np.zeros((768, 8))
    with pytest.raises(ValueError):
        oracle.bsa_slice_ref(q, q, q, np.ones((768, 3)), 16, 0, 32)
    with pytest.raises(ValueError):
        oracle.bsa_slice_ref(q, q, q, np.ones((768, 3)), 16, 49, 32)
    with pytest.raises(ValueError):
        oracle.bsa_slice_ref(q, q, q, np.ones((768, 3)), 16, 4, 0)
    with pytest.raises(ValueError):
        oracle.bsa_slice_ref(q[:700], q[:700], q[:700], np.ones((700, 3)), 4, 4, 32)
