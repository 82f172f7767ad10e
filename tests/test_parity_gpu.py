"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every case prints its name, shape and seed before it touches the GPU.
Small workloads are compared element by element on every slice; the
Nside = 128 and 256 workloads run in the bench's launch configuration
(whole batch, one forward call) and are compared on all index rows of a
sample of slices and on sampled output tokens.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import CONFIGS, BSAConfig, make_inputs
from spherical_block_sparse_amd import _lib
from spherical_block_sparse_amd.synth import to_f64

from parity import assert_close, check_indices, log, ocg_tolerance, selection_ref

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _gpu_inputs(cfg: BSAConfig, seed=None):
    log(f"[case] {cfg.name}: nside={cfg.nside} b={cfg.batch} H={cfg.heads} d={cfg.head_dim} "
        f"block={cfg.block} topn={cfg.topn} W={cfg.window} field={cfg.field} seed={cfg.seed if seed is None else seed}")
    return make_inputs(cfg, device=DEV, dtype=torch.bfloat16, seed=seed)


def _slice(x, b, h):
    return to_f64(x[b, h])


def _full_compare(cfg, q, k, v, g, out, idx, slices=None):
    """Compare indices and every output element of the listed slices."""
    stats = []
    for (b, h) in (slices or [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]):
        qs, ks, vs, gs = _slice(q, b, h), _slice(k, b, h), _slice(v, b, h), _slice(g, b, h)
        ref_sel = selection_ref(qs, ks, vs, cfg.block, cfg.topn)
        gi = idx[b, h].cpu().numpy()
        st = check_indices(gi, ref_sel, cfg.topn)
        ref = oracle.bsa_slice_ref(qs, ks, vs, gs, cfg.block, cfg.topn, cfg.window, idx=gi)
        assert_close(out[b, h].cpu().numpy(), ref["out"], f"out[{b},{h}] (near-ties {st['near_ties']})")
        stats.append(st)
    return stats


# ------------------------------------------------------------------ stages --

@pytest.mark.parametrize("name", ["tiny", "ns32"])
def test_pool_stage_bit_exact(name):
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block)
    torch.cuda.synchronize()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            np.testing.assert_array_equal(qbar[b, h].cpu().numpy(), oracle.pool_mean(_slice(q, b, h), cfg.block))
            np.testing.assert_array_equal(kbar[b, h].cpu().numpy(), oracle.pool_mean(_slice(k, b, h), cfg.block))
            np.testing.assert_array_equal(vbar[b, h].cpu().numpy(),
                                          oracle.pool_mean(_slice(v, b, h), cfg.block).astype(np.float32))


@pytest.mark.parametrize("name", ["tiny", "ns32", "ns64"])
def test_compress_select_stage(name):
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    torch.cuda.synchronize()
    near = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = selection_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h), cfg.block, cfg.topn)
            near += check_indices(sel[b, h].cpu().numpy(), ref, cfg.topn)["near_ties"]
            np.testing.assert_allclose(o_cg[b, h].cpu().numpy(), ref["o_cg"], rtol=0, atol=ocg_tolerance(ref["vbar"]))
    log(f"    indices: {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")


def _check_compress_select(cfg, q, k, v, topn=None):
    topn = topn or cfg.topn
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, topn)
    torch.cuda.synchronize()
    near = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = selection_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h), cfg.block, topn)
            near += check_indices(sel[b, h].cpu().numpy(), ref, topn)["near_ties"]
            np.testing.assert_allclose(o_cg[b, h].cpu().numpy(), ref["o_cg"], rtol=0, atol=ocg_tolerance(ref["vbar"]))
    return near


def test_compress_select_rows_crowded_into_one_lane_group():
    """Key blocks j = 0 mod 4 carry a large common direction u, and the query
    blocks i = 0 mod 3 carry it too: those rows' whole top-16 sits in blocks
    congruent mod 4, i.e. in the share of the keys one lane of the selection
    sees, so that lane's list must hold all of them."""
    cfg = CONFIGS["ns32"]
    q, k, v, _ = _gpu_inputs(cfg)
    gen = torch.Generator(device="cpu").manual_seed(5)
    u = torch.randn(cfg.head_dim, generator=gen, dtype=torch.float64)
    u = (3.0 * u / u.norm()).to(DEV)
    B, m = cfg.block, cfg.n_blocks
    kb = (torch.arange(cfg.n_tokens, device=DEV) // B) % 4 == 0
    qb = (torch.arange(cfg.n_tokens, device=DEV) // B) % 3 == 0
    k = (k.double() + kb[:, None] * u).bfloat16()
    q = (q.double() + qb[:, None] * u).bfloat16()
    near = _check_compress_select(cfg, q, k, v)
    log(f"    {cfg.slices * m} rows ({cfg.slices * ((m + 2) // 3)} crowded), {near} near-tie rows")


@pytest.mark.parametrize("topn", [17, 32, 64])
def test_compress_select_topn_above_sixteen(topn):
    cfg = CONFIGS["ns32"]
    q, k, v, _ = _gpu_inputs(cfg)
    _check_compress_select(cfg, q, k, v, topn=topn)


def _knorm(cfg):
    return torch.empty((cfg.batch, cfg.heads, cfg.n_blocks), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("name", ["tiny", "ns32"])
def test_pool_block_max_key_norm(name):
    """The pool's largest key norm per block is max_t |k_t| over the block's tokens, up to float32
    rounding of the sums of squares (the datum the fine kernel's score bounds come from)."""
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    knorm = _knorm(cfg)
    _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    torch.cuda.synchronize()
    want = k.double().cpu().norm(dim=-1).reshape(cfg.batch, cfg.heads, cfg.n_blocks, -1).amax(-1)
    got = knorm.double().cpu()
    assert torch.all((got - want).abs() <= 1e-5 * want), (got - want).abs().max().item()


@pytest.mark.parametrize("bounds", [False, True])
@pytest.mark.parametrize("name", ["tiny", "ns32"])
def test_fine_stage_branches_one_hot(name, bounds):
    """mosaic_bsa_fine with one-hot gates isolates o_CG, o_FG and o_L, with the running-maximum
    softmax (no knorm) and with the pool's score bounds."""
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    knorm = _knorm(cfg) if bounds else None
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    for col, key in [(0, "o_cg"), (1, "o_fg"), (2, "o_l")]:
        g = torch.zeros((cfg.batch, cfg.heads, cfg.n_tokens, 3), dtype=torch.float32, device=DEV)
        g[..., col] = 1.0
        out = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                   knorm=knorm)
        torch.cuda.synchronize()
        for b in range(cfg.batch):
            for h in range(min(cfg.heads, 2)):
                gi = sel[b, h].cpu().numpy()
                ref = oracle.bsa_slice_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h),
                                           np.ones((cfg.n_tokens, 3)), cfg.block, cfg.topn, cfg.window, idx=gi)
                want = ref[key][np.arange(cfg.n_tokens) // cfg.block] if key == "o_cg" else ref[key]
                assert_close(out[b, h].cpu().numpy(), want, f"{key}[{b},{h}]")


# blocks of 256 tokens: the fine kernel runs 128-query tiles on 4 waves
WIDE = CONFIGS["ns32"].with_(name="ns16-b256", nside=16, block=256, topn=4, window=100, batch=2, heads=2, seed=16)


def test_forward_wide_tiles_all_slices():
    """Blocks of 256 tokens (4-wave, 128-query fine tiles) at a size the oracle runs in full."""
    cfg = WIDE
    q, k, v, g = _gpu_inputs(cfg)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    _full_compare(cfg, q, k, v, g, out, idx)


@pytest.mark.parametrize("name,scale", [("tiny", 1.0), ("tiny", 3.5), ("tiny", 8.0),
                                        ("ns32", 1.0), ("ns32", 3.0), ("ns32", 4.0),
                                        ("wide", 1.0), ("wide", 4.0)])
def test_fine_score_bound_paths(name, scale):
    """q scaled (and rounded back to bf16) so that the score bounds c*|q|*max|k| from the pool's
    largest key norms are small for every wave (all take the bound as their fixed reference:
    tiny and ns32 unscaled), small for some waves only (tiny at 3.5, ns32 at 3), or too large
    everywhere (the running maximum: tiny at 8, ns32 at 4).  The output matches the oracle in
    each case, with and without knorm."""
    cfg = WIDE if name == "wide" else CONFIGS[name]
    q, k, v, g = _gpu_inputs(cfg)
    q = (q.float() * scale).to(torch.bfloat16)
    log(f"[case] q scaled by {scale}")
    knorm = _knorm(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    out_b = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm)
    out_l = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (cfg.batch - 1, cfg.heads - 1)]:
        gi = sel[b, h].cpu().numpy()
        ref = oracle.bsa_slice_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h), _slice(g, b, h),
                                   cfg.block, cfg.topn, cfg.window, idx=gi)
        assert_close(out_b[b, h].cpu().numpy(), ref["out"], f"bounded out[{b},{h}]")
        assert_close(out_l[b, h].cpu().numpy(), ref["out"], f"running-max out[{b},{h}]")


# ---------------------------------------------------------- end to end ------

@pytest.mark.parametrize("name", ["tiny", "ns32"])
def test_forward_all_slices(name):
    cfg = CONFIGS[name]
    q, k, v, g = _gpu_inputs(cfg)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    _full_compare(cfg, q, k, v, g, out, idx)


def test_forward_ns64_indices_all_outputs_two_slices():
    cfg = CONFIGS["ns64"]
    q, k, v, g = _gpu_inputs(cfg)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    near = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = selection_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h), cfg.block, cfg.topn)
            near += check_indices(idx[b, h].cpu().numpy(), ref, cfg.topn)["near_ties"]
    log(f"    indices: {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")
    _full_compare(cfg, q, k, v, g, out, idx, slices=[(0, 0), (cfg.batch - 1, cfg.heads - 1)])


def _sampled_full_size(cfg: BSAConfig, n_slices=4, n_tokens=192):
    q, k, v, g = _gpu_inputs(cfg)
    need = _lib.mosaic_bsa_workspace_bytes(cfg.batch, cfg.heads, cfg.head_dim, cfg.nside, cfg.block, cfg.topn)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(cfg.seed)
    S = cfg.slices
    picks = sorted(set([0, S - 1] + list(rng.choice(S, n_slices - 2, replace=False))))
    N, B = cfg.n_tokens, cfg.block
    errs, refs = [], []
    for sidx in picks:
        b, h = divmod(int(sidx), cfg.heads)
        qs, ks, vs, gs = _slice(q, b, h), _slice(k, b, h), _slice(v, b, h), _slice(g, b, h)
        ref_sel = selection_ref(qs, ks, vs, B, cfg.topn)
        gi = idx[b, h].cpu().numpy()
        st = check_indices(gi, ref_sel, cfg.topn)
        toks = np.unique(np.concatenate([np.arange(64), N - 64 + np.arange(64),
                                         rng.choice(N, n_tokens, replace=False),
                                         B * rng.choice(N // B, 8, replace=False)]))
        r = oracle.bsa_rows_ref(qs, ks, vs, gs, B, cfg.topn, cfg.window, toks, idx=gi)
        got = out[b, h].cpu().numpy()[toks]
        assert_close(got, r["out"], f"slice ({b},{h}) {toks.size} tokens, {st['rows']} idx rows, "
                                    f"{st['near_ties']} near-ties")
        errs.append(got - r["out"])
        refs.append(r["out"])
    assert_close(np.concatenate(errs) + np.concatenate(refs), np.concatenate(refs), "all sampled tokens")


def test_forward_ns128_full_size_sampled():
    _sampled_full_size(CONFIGS["ns128"])


def test_forward_ns256_full_size_sampled():
    _sampled_full_size(CONFIGS["ns256"])


# ------------------------------------------------------------- edge cases ---

def _edge(cfg: BSAConfig, mutate=None, window=None, topn=None, gates=None, check_out=True):
    cfg = cfg.with_(window=window or cfg.window, topn=topn or cfg.topn)
    q, k, v, g = _gpu_inputs(cfg)
    if mutate:
        q, k, v = mutate(q, k, v)
    if gates is not None:
        g = gates(g)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    if check_out:
        _full_compare(cfg, q, k, v, g, out, idx)
    return cfg, q, k, v, g, out, idx


def test_edge_topn_all_blocks():
    cfg, *_ , idx = _edge(CONFIGS["tiny"], topn=48)
    assert torch.equal(idx.cpu(), torch.arange(48, dtype=torch.int32).expand(1, 2, 48, 48))


def test_edge_topn_one():
    _edge(CONFIGS["tiny"], topn=1)


def test_edge_window_one_is_v():
    g1 = lambda g: torch.zeros_like(g).index_fill_(-1, torch.tensor([2], device=DEV), 1.0)
    cfg, q, k, v, g, out, idx = _edge(CONFIGS["tiny"], window=1, gates=g1)
    # o_L is v itself; the one weight w need not be exactly 1 (a score bound can be the softmax
    # reference), so out = (1/w)(w v) is v up to float32 rounding of that product and quotient
    want = v.float()
    assert torch.all((out - want).abs() <= 2 * 2.0 ** -23 * want.abs())


def test_edge_window_wider_than_sphere():
    _edge(CONFIGS["tiny"], window=10 ** 6)


def test_edge_odd_window():
    _edge(CONFIGS["tiny"], window=33)


def test_edge_zero_block_means_give_lowest_indices():
    """q alternating in sign inside each block: q̄ = 0, every logit is exactly
    0, so the selection must be blocks 0..n-1 (lower-index tie rule)."""
    def mutate(q, k, v):
        q = q.clone()
        q[:, :, 1::2] = -q[:, :, 0::2]
        return q, k, v
    cfg, q, k, v, g, out, idx = _edge(CONFIGS["tiny"], mutate=mutate)
    assert torch.equal(idx.cpu(), torch.arange(4, dtype=torch.int32).expand(1, 2, 48, 4))


def test_edge_zero_queries_uniform_weights():
    cfg, q, k, v, g, out, idx = _edge(CONFIGS["tiny"], mutate=lambda q, k, v: (torch.zeros_like(q), k, v))
    assert torch.equal(idx.cpu(), torch.arange(4, dtype=torch.int32).expand(1, 2, 48, 4))


def test_edge_block_constant_inputs_exact_ties():
    """Every block holds one repeated token: many equal k̄ rows -> exact ties."""
    def mutate(q, k, v):
        rep = lambda x: x[:, :, ::16].repeat_interleave(16, dim=2).contiguous()
        kk = rep(k)
        kk[:, :, 16 * 10:16 * 20] = kk[:, :, 0:16].repeat(1, 1, 10, 1)   # ten copies of block 0
        return rep(q), kk, rep(v)
    _edge(CONFIGS["tiny"], mutate=mutate)


def test_edge_head_dim_64_block_16():
    _edge(CONFIGS["tiny"].with_(name="tiny-d64", head_dim=64, heads=3, batch=2))


def test_edge_block_256_ragged_chunks():
    # nside 16: N = 3072, m = 12 blocks of 256, topn 3 -> 768 selected keys
    _edge(BSAConfig("n16-b256", 16, 1, 2, 64, 256, 3, 100, "iid", 16))


def test_edge_head_dim_32_block_256():
    # 128-query tiles with head_dim 32
    _edge(BSAConfig("n16-b256-d32", 16, 1, 2, 32, 256, 3, 100, "iid", 17))


def test_edge_block_64_small_m():
    # nside 8 with block 64: m = 12 (< one 64-row tile), window > N/2
    _edge(BSAConfig("n8-b64", 8, 2, 2, 32, 64, 5, 500, "iid", 9))


def test_edge_large_logits():
    """Scaled inputs: peaked softmaxes in every branch."""
    _edge(CONFIGS["tiny"].with_(name="tiny-x4"), mutate=lambda q, k, v: ((q.float() * 4).bfloat16(), k, v))


def test_determinism_bitwise():
    cfg = CONFIGS["ns32"]
    q, k, v, g = _gpu_inputs(cfg)
    o1, i1 = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    o2, i2 = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(i1, i2)


def test_forward_equals_stages():
    cfg = CONFIGS["ns32"]
    q, k, v, g = _gpu_inputs(cfg)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    knorm = _knorm(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    out2 = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm)
    torch.cuda.synchronize()
    assert torch.equal(idx, sel) and torch.equal(out, out2)
