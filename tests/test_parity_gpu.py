"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every case prints its name, shape and seed before it touches the GPU.
Small workloads are compared element by element on every slice.  The
Nside = 64, 128 and 256 workloads run in the bench's launch configuration
(whole batch, one forward call); every index row of every slice is checked,
and every output element of all ns64 slices and of 8 seeded slices at
ns128 and ns256 (the oracle runs in a pool of host processes).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import CONFIGS, BSAConfig, make_inputs
from spherical_block_sparse_amd import _lib
from spherical_block_sparse_amd.locality_study import permute_tokens
from spherical_block_sparse_amd.synth import nest_ring_order, to_f64

import oracle_jobs
from parity import MAX_ABS, NEAR_TIE, REL_L2, assert_close, check_indices, log, ocg_tolerance, selection_ref

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


def _pieces(cfg):
    """Buffers for the pool's bf16 pieces of k̄ and |k̄_j|^2."""
    return (torch.empty((cfg.batch, cfg.heads, cfg.n_blocks, 2, cfg.head_dim), dtype=torch.bfloat16, device=DEV),
            torch.empty((cfg.batch, cfg.heads, cfg.n_blocks), dtype=torch.float32, device=DEV))


def _check_compress_select(cfg, q, k, v, topn=None, pieces=False):
    """Selection bit-exact (outside near ties) and o_CG within its bound, with the float64
    logits (pieces False) or the certified bf16-piece logits (pieces True)."""
    topn = topn or cfg.topn
    kp, kb2 = _pieces(cfg) if pieces else (None, None)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, kpieces=kp, kbn2=kb2)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, topn, kpieces=kp, kbn2=kb2)
    torch.cuda.synchronize()
    near = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = selection_ref(_slice(q, b, h), _slice(k, b, h), _slice(v, b, h), cfg.block, topn)
            near += check_indices(sel[b, h].cpu().numpy(), ref, topn)["near_ties"]
            np.testing.assert_allclose(o_cg[b, h].cpu().numpy(), ref["o_cg"], rtol=0, atol=ocg_tolerance(ref["vbar"]))
    return near


@pytest.mark.parametrize("pieces", [False, True], ids=["f64", "pieces"])
@pytest.mark.parametrize("name", ["tiny", "ns32", "ns64"])
def test_compress_select_stage(name, pieces):
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    near = _check_compress_select(cfg, q, k, v, pieces=pieces)
    log(f"    indices: {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")


@pytest.mark.parametrize("name", ["tiny", "ns32"])
def test_pool_key_pieces(name):
    """The pool's pieces of k̄ are k1 = bf16(float32(k̄)) and k2 = bf16(float32(k̄) - k1), with
    k̄ the oracle's block mean (rounding to nearest even, as torch rounds), and its |k̄_j|^2 is
    the float64 sum of squares rounded up by at most 2e-6 relative."""
    cfg = CONFIGS[name]
    q, k, v, _ = _gpu_inputs(cfg)
    kp, kb2 = _pieces(cfg)
    _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, kpieces=kp, kbn2=kb2)
    torch.cuda.synchronize()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            kbar = torch.from_numpy(oracle.pool_mean(_slice(k, b, h), cfg.block))
            xf = kbar.float()
            k1 = xf.bfloat16()
            k2 = (xf - k1.float()).bfloat16()
            got = kp[b, h].cpu()
            assert torch.equal(got[:, 0].view(torch.int16), k1.view(torch.int16))
            assert torch.equal(got[:, 1].view(torch.int16), k2.view(torch.int16))
            n2 = (kbar * kbar).sum(-1)
            g2 = kb2[b, h].double().cpu()
            assert torch.all(g2 >= n2) and torch.all(g2 <= n2 * (1 + 2e-6))


@pytest.mark.parametrize("share", [1.0, 0.25], ids=["all", "quarter"])
def test_compress_select_pieces_massive_ties(share):
    """Key blocks with identical k̄ (every key block, or one in four) give rows whose n-th logit
    is shared by more keys than the certified band holds: the workgroup settles those rows with
    its exact float64 fallback, so the lower-index rule still decides."""
    cfg = CONFIGS["ns32"]
    q, k, v, _ = _gpu_inputs(cfg)
    B = cfg.block
    blk = torch.arange(cfg.n_tokens, device=DEV) // B
    same = (blk % 4 == 0) if share < 1 else torch.ones_like(blk, dtype=torch.bool)
    # every chosen block repeats the first block's tokens of its slice
    k = torch.where(same[None, None, :, None], k[:, :, :B].repeat(1, 1, cfg.n_tokens // B, 1), k)
    near = _check_compress_select(cfg, q, k, v, pieces=True)
    log(f"    {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")


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
    for pieces in (False, True):
        near = _check_compress_select(cfg, q, k, v, pieces=pieces)
        log(f"    {cfg.slices * m} rows ({cfg.slices * ((m + 2) // 3)} crowded), {near} near-tie rows, "
            f"pieces {pieces}")


@pytest.mark.parametrize("block", [64, 1], ids=["cached", "uncached"])
def test_compress_select_pieces_exact_rows(block):
    """A few rows per row tile that the certification cannot settle, so that the workgroup
    selects them exactly itself: query blocks of slice 0 set to zero, one per row tile or
    fewer, have every logit equal to 0, so the lower-index rule gives blocks 0 .. n-1.  Blocks
    of 64 tokens at Nside 32 (m = 192: the logits fit the LDS cache) and blocks of one token
    (m = 12288: recomputed on every radix pass).  Those rows and every 8th row of slice 0 are
    checked against the oracle."""
    cfg = CONFIGS["ns32"].with_(name=f"ns32-b{block}", block=block, heads=1 if block == 1 else 8, topn=16,
                                seed=321 + block)
    q, k, v, _ = _gpu_inputs(cfg)
    m, B = cfg.n_blocks, cfg.block
    qblocks = torch.arange(5, m, 96 if m < 1024 else 768)[:16]
    tok = (qblocks[:, None] * B + torch.arange(B)[None, :]).reshape(-1).to(DEV)
    q[0, 0, tok] = 0
    kp, kb2 = _pieces(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, kpieces=kp, kbn2=kb2)
    _, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn, kpieces=kp,
                                             kbn2=kb2)
    torch.cuda.synchronize()
    qb = oracle.pool_mean(_slice(q, 0, 0), B)
    kb = oracle.pool_mean(_slice(k, 0, 0), B)
    rows = np.union1d(np.arange(0, m, 8), qblocks.numpy())
    idx, gap = oracle.select_topn(qb[rows] @ kb.T, cfg.topn)
    got = sel[0, 0].cpu().numpy()[rows]
    exact = ~((gap > 0) & (gap < 1e-6))
    assert np.array_equal(got[exact], idx[exact])
    zero = np.isin(rows, qblocks.numpy())
    assert np.array_equal(got[zero], np.tile(np.arange(cfg.topn), (int(zero.sum()), 1)))
    log(f"    {rows.size} rows checked ({int(zero.sum())} zero-query rows), {int((~exact).sum())} near ties")


@pytest.mark.parametrize("topn", [1, 3, 8, 13, 16])
def test_compress_select_pieces_topn(topn):
    """The certified approximate ranking at every list depth it serves (n <= 16)."""
    cfg = CONFIGS["ns32"]
    q, k, v, _ = _gpu_inputs(cfg)
    near = _check_compress_select(cfg, q, k, v, topn=topn, pieces=True)
    log(f"    topn {topn}: {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")


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
    sb = _lib.mosaic_bsa_select_bound(sel, knorm, cfg.nside, cfg.block, cfg.topn, cfg.head_dim)
    out_s = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm,
                                 sel_bound=sb)
    torch.cuda.synchronize()
    assert torch.equal(out_b, out_s)     # the precomputed bound is the one the kernel gathers
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


def _bits(x):
    """Host copy of a bf16 device tensor as its uint16 bit patterns."""
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def _full_size(cfg: BSAConfig, n_out_slices=None, ring=False):
    """The workload in the bench's launch configuration (whole batch, one
    forward call): every index row of every slice against the oracle's
    selection, and every output element of ``n_out_slices`` seeded slices
    (first and last included; all slices when None) against the oracle run
    with the GPU's indices.  The oracle runs in a pool of host processes.
    ``ring`` lays the same field out in RING (iso-latitude) token order."""
    q, k, v, g = _gpu_inputs(cfg)
    if ring:
        q, k, v, g = permute_tokens([q, k, v, g], nest_ring_order(cfg.nside))
    need = _lib.mosaic_bsa_workspace_bytes(cfg.batch, cfg.heads, cfg.head_dim, cfg.nside, cfg.block, cfg.topn)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out, idx = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    S = cfg.slices
    if n_out_slices is None or n_out_slices >= S:
        out_slices = set(range(S))
    else:
        rng = np.random.default_rng(cfg.seed)
        out_slices = {0, S - 1} | set(int(x) for x in rng.choice(np.arange(1, S - 1), n_out_slices - 2, replace=False))
    log(f"    oracle on {oracle_jobs.workers()} host processes: {S} slices of index rows, "
        f"{len(out_slices)} whole output slices {sorted(out_slices)}")
    pending = []
    with oracle_jobs.pool() as pool:
        for sidx in range(S):
            b, h = divmod(sidx, cfg.heads)
            qb, kb, vb, gi = _bits(q[b, h]), _bits(k[b, h]), _bits(v[b, h]), idx[b, h].cpu().numpy()
            pending.append(pool.apply_async(oracle_jobs.index_job,
                                            ((b, h), qb, kb, vb, cfg.block, cfg.topn, gi)))
            if sidx in out_slices:
                pending.append(pool.apply_async(oracle_jobs.output_job,
                                                ((b, h), qb, kb, vb, g[b, h].cpu().numpy(), cfg.block, cfg.topn,
                                                 cfg.window, gi, out[b, h].cpu().numpy())))
        del q, k, v, g, out
        rows = near = n_out = 0
        diff2 = ref2 = worst = 0.0
        for i, res in enumerate(pending):
            r = res.get()
            if "ok" in r:
                assert r["ok"], f"slice {r['tag']}: {r['msg']}"
                rows += r["rows"]
                near += r["near_ties"]
            else:
                assert r["finite"], f"slice {r['tag']}: non-finite output"
                assert r["max_abs"] <= MAX_ABS and r["rel"] <= REL_L2, \
                    f"slice {r['tag']}: max-abs {r['max_abs']:.3e} rel-L2 {r['rel']:.3e}"
                n_out += 1
                diff2 += r["diff2"]
                ref2 += r["ref2"]
                worst = max(worst, r["max_abs"])
            if (i + 1) % 32 == 0 or i + 1 == len(pending):
                log(f"    {i + 1}/{len(pending)} oracle jobs checked")
    rel = (diff2 / ref2) ** 0.5
    log(f"    indices: {rows} rows ({S} slices x {cfg.n_blocks}), all bit-exact except {near} near-tie rows "
        f"(checked top-{cfg.topn} within {NEAR_TIE:g})")
    log(f"    outputs: {n_out} whole slices, max-abs {worst:.3e}, rel-L2 over them {rel:.3e}")
    assert rows == S * cfg.n_blocks and n_out == len(out_slices)
    assert rel <= REL_L2


def test_forward_ns64_every_slice():
    """ns64: every index row and every output element of all 32 slices."""
    _full_size(CONFIGS["ns64"])


def test_forward_ns64_ring_order_every_row():
    """The ns64 field in RING token order: a block is then a strip of one
    iso-latitude ring, and the logits of neighbouring strips crowd within
    the approximate selection's error bound on many rows, so the exact
    in-workgroup fallback and the float64 redo of crowded tiles carry much
    of the selection.  Every index row of all 32 slices, and 4 whole output
    slices, against the oracle."""
    _full_size(CONFIGS["ns64"], n_out_slices=4, ring=True)


def test_forward_ns128_full_size():
    """ns128 (the bench workload): every index row of the 192 slices, whole outputs of 8 slices."""
    _full_size(CONFIGS["ns128"], n_out_slices=8)


def test_forward_ns256_full_size():
    """ns256: every index row of the 32 slices, whole outputs of 8 slices."""
    _full_size(CONFIGS["ns256"], n_out_slices=8)


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
    kp, kb2 = _pieces(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm, kpieces=kp, kbn2=kb2)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn, kpieces=kp,
                                                kbn2=kb2)
    out2 = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm)
    sb = _lib.mosaic_bsa_select_bound(sel, knorm, cfg.nside, cfg.block, cfg.topn, cfg.head_dim)
    out3 = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm,
                                sel_bound=sb)
    torch.cuda.synchronize()
    assert torch.equal(idx, sel) and torch.equal(out, out2) and torch.equal(out, out3)
    # the bound is a maximum of stored values: exact
    want = torch.gather(knorm.unsqueeze(2).expand(-1, -1, cfg.n_blocks, -1), 3, sel.long()).amax(dim=3)
    assert torch.equal(sb, want)


# ------------------------------- blocks of 1 and 4 tokens, top-n above 64 ---
# These shapes run the one-wave-per-row kernels (generic selection when
# topn > 64, generic fine attention when block < 16 or the tiled kernel's
# selection table would overflow) and the pool's one-row sweep.

B1 = CONFIGS["tiny"].with_(name="tiny-b1", block=1, seed=81)
B4 = CONFIGS["tiny"].with_(name="tiny-b4", block=4, seed=84)


@pytest.mark.parametrize("cfg", [B1, B4], ids=lambda c: c.name)
def test_pool_small_blocks_bit_exact_and_key_norms(cfg):
    q, k, v, _ = _gpu_inputs(cfg)
    knorm = _knorm(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    torch.cuda.synchronize()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            np.testing.assert_array_equal(qbar[b, h].cpu().numpy(), oracle.pool_mean(_slice(q, b, h), cfg.block))
            np.testing.assert_array_equal(kbar[b, h].cpu().numpy(), oracle.pool_mean(_slice(k, b, h), cfg.block))
            np.testing.assert_array_equal(vbar[b, h].cpu().numpy(),
                                          oracle.pool_mean(_slice(v, b, h), cfg.block).astype(np.float32))
    want = k.double().cpu().norm(dim=-1).reshape(cfg.batch, cfg.heads, cfg.n_blocks, -1).amax(-1)
    assert torch.all((knorm.double().cpu() - want).abs() <= 1e-5 * want)


def test_block_one_compressed_branch_is_dense_attention():
    """Blocks of one token: q̄, k̄, v̄ are q, k, v, so o_CG is dense softmax
    attention over the whole sphere (torch float64 here, independent of the
    oracle); then the whole forward against the oracle."""
    cfg = B1
    q, k, v, g = _gpu_inputs(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block)
    o_cg, _ = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    torch.cuda.synchronize()
    qd, kd, vd = (x.double().cpu() for x in (q, k, v))
    dense = torch.softmax(qd @ kd.transpose(-1, -2) / cfg.head_dim ** 0.5, dim=-1) @ vd
    tol = ocg_tolerance(vd.numpy())
    err = float((o_cg.double().cpu() - dense).abs().max())
    log(f"    o_CG vs dense attention: max-abs {err:.3e} (bound {tol:.3e})")
    assert err <= tol
    _edge(cfg)


def test_block_four_forward():
    _edge(B4)


def test_block_four_forward_save_state():
    """mosaic_bsa_forward_train on blocks of 4 (generic fine kernel, SAVE
    outputs): the same out and selection as the forward, and the saved
    normalised branch outputs against the oracle's branches."""
    cfg = B4
    q, k, v, g = _gpu_inputs(cfg)
    out0, sel0 = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    out, sel, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel0)
    assert float((out - out0).abs().max()) <= 1e-6 * float(out0.abs().max())
    S, N, d = cfg.slices, cfg.n_tokens, cfg.head_dim
    o = saved[:S * N * 2 * d * 4].view(torch.float32).view(cfg.batch, cfg.heads, N, 2, d)
    for h in range(cfg.heads):
        qs, ks, vs = _slice(q, 0, h), _slice(k, 0, h), _slice(v, 0, h)
        gi = sel[0, h].cpu().numpy()
        assert_close(o[0, h, :, 0].cpu().numpy(), oracle.fine_selected_branch(qs, ks, vs, gi, cfg.block), f"o_FG[{h}]")
        assert_close(o[0, h, :, 1].cpu().numpy(), oracle.local_branch(qs, ks, vs, cfg.window), f"o_L[{h}]")


def test_topn_all_blocks_ns32():
    """top-n = m = 192 (the exact radix selection): every row selects every
    block, and the selected branch is dense attention."""
    cfg, *_, idx = _edge(CONFIGS["ns32"].with_(name="ns32-all", heads=2), topn=192)
    assert torch.equal(idx.cpu(), torch.arange(192, dtype=torch.int32).expand(1, 2, 192, 192))


@pytest.mark.parametrize("topn", [65, 100, 191])
def test_compress_select_stage_any_topn(topn):
    cfg = CONFIGS["ns32"]
    q, k, v, _ = _gpu_inputs(cfg)
    near = _check_compress_select(cfg, q, k, v, topn=topn)
    log(f"    topn {topn}: {cfg.slices * cfg.n_blocks} rows, {near} near-tie rows")


# nside 16, blocks of 16 (m = 192): top-100 overflows the tiled kernel's selection table
N16 = BSAConfig("n16-b16-top100", 16, 1, 3, 64, 16, 100, 64, "iid", 161)


def test_topn_above_the_tile_table():
    _edge(N16)


def test_topn_above_64_exact_ties():
    """Block-constant inputs with repeated key blocks: exact ties in the
    radix selection go to the lower block index."""
    def mutate(q, k, v):
        rep = lambda x: x[:, :, ::16].repeat_interleave(16, dim=2).contiguous()
        kk = rep(k)
        kk[:, :, 16 * 20:16 * 60] = kk[:, :, 0:16].repeat(1, 1, 40, 1)   # forty copies of block 0
        return rep(q), kk, rep(v)
    _edge(N16.with_(name="n16-top100-ties"), mutate=mutate)


def test_block_four_top80_ns32():
    """Blocks of 4 on the Nside-32 mesh (m = 3072), top-80: the radix
    selection over 3072 keys per row and the generic fine kernel."""
    _edge(CONFIGS["ns32"].with_(name="ns32-b4-top80", block=4, topn=80, heads=2, seed=324))


def test_block_one_ns32_one_head():
    """Blocks of one token on the Nside-32 mesh: m = N = 12288 rows in the
    lane-list selection, the generic fine kernel on 16 single-token blocks
    plus the window."""
    _edge(CONFIGS["ns32"].with_(name="ns32-b1", block=1, heads=1, seed=321))


# The smallest spheres: Nside 1 (the 12 base pixels, blocks of one token,
# m = 12) and Nside 2 (48 tokens, blocks of 1 or 4), so that a row tile, a
# key chunk and a window are each larger than the whole sphere.
SMALLEST = [
    BSAConfig("s1-b1-top1-w1", 1, 2, 2, 64, 1, 1, 1, "iid", 101),
    BSAConfig("s1-b1-top12-w12-d32", 1, 2, 2, 32, 1, 12, 12, "iid", 102),
    BSAConfig("s1-b1-top5-w7", 1, 2, 2, 64, 1, 5, 7, "iid", 103),
    BSAConfig("s2-b4-top12-w48", 2, 2, 2, 64, 4, 12, 48, "iid", 104),
    BSAConfig("s2-b4-top3-w5-d32", 2, 2, 2, 32, 4, 3, 5, "iid", 105),
    BSAConfig("s2-b1-top48-w20", 2, 2, 2, 64, 1, 48, 20, "iid", 106),
    BSAConfig("s2-b1-top20-w9", 2, 2, 2, 64, 1, 20, 9, "iid", 107),
]


@pytest.mark.parametrize("cfg", SMALLEST, ids=lambda c: c.name)
def test_edge_smallest_spheres(cfg):
    _, *_, idx = _edge(cfg)
    if cfg.topn == cfg.n_blocks:   # every row selects every block, in ascending order
        want = torch.arange(cfg.n_blocks, dtype=torch.int32).expand(cfg.batch, cfg.heads, cfg.n_blocks, cfg.n_blocks)
        assert torch.equal(idx.cpu(), want)


@pytest.mark.parametrize("cfg", [B1, B4, CONFIGS["ns32"].with_(name="ns32-b16-top80", block=16, heads=2, topn=80,
                                                                 seed=325),
                                 CONFIGS["ns32"].with_(name="ns32-top80", heads=2, topn=80, seed=326)],
                         ids=lambda c: c.name)
def test_select_bound_beyond_the_forward_shapes(cfg):
    """mosaic_bsa_select_bound where the fine attention runs the one-wave kernel (blocks of 1 or 4
    tokens; 4 query blocks of 16 tokens x 80 selected overflow the tiled kernel's table), which
    forms its references itself, and where the tiled kernel reads it with top-n above 64 (blocks of
    64): the bound is the exact maximum of the selected blocks' norms, and the fine stage given it
    is bit-identical to the stage without it."""
    q, k, v, g = _gpu_inputs(cfg)
    knorm = _knorm(cfg)
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
    sb = _lib.mosaic_bsa_select_bound(sel, knorm, cfg.nside, cfg.block, cfg.topn, cfg.head_dim)
    out_a = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm)
    out_b = _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm,
                                 sel_bound=sb)
    torch.cuda.synchronize()
    want = torch.gather(knorm.unsqueeze(2).expand(-1, -1, cfg.n_blocks, -1), 3, sel.long()).amax(dim=3)
    assert torch.equal(sb, want)
    assert torch.equal(out_a, out_b)
