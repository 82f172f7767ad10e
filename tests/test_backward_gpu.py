"""GPU parity of mosaic_bsa_backward against the float64 oracle backward
(``oracle.bsa_backward``), through the C ABI.

Both sides take the same bf16 inputs (the oracle on their float64 values),
the same float32 dout and the same selection (the GPU forward's indices,
which the backward holds fixed), so the comparison is element by element.

Tolerance, from the arithmetic of the kernels: every product is bf16 x bf16
with float32 accumulation; q, k, v are exact bf16 inputs, while dout, the
probabilities P|g| and dS = P g (dP - dO_b·o) are rounded to bf16 (relative error
<= 2^-9 each) before they enter a product.  D is formed from the same
bf16 dout as dP, so a row's dS still sums to zero up to rounding and no
systematic error times the mean key enters dQ or dK.  A gradient element is
a sum of such rounded terms, so its error is a few 2^-9 relative to the sum
of the magnitudes of its terms, not to its (possibly cancelling) value.  The
check is relative L2 per tensor <= 1e-2 and max-abs <= 2e-2 times the
tensor's largest magnitude (measured: <= 4e-3 and <= 5e-3).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import BSAConfig, _lib, make_inputs
from spherical_block_sparse_amd.synth import to_f64

from parity import log

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2


def _run(cfg: BSAConfig, seed: int = 0, gates=None, use_saved: bool = False):
    dev = "cuda"
    q, k, v, g = make_inputs(cfg, device=dev)
    if gates is not None:
        g = gates(g)
    gen = torch.Generator(device=dev).manual_seed(1000 + cfg.seed + seed)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32)
    saved = None
    if use_saved:
        _, sel, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    else:
        _, sel = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    dq, dk, dv, dg = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                              saved=saved)
    torch.cuda.synchronize()
    ref = oracle.bsa_backward_ref(to_f64(q), to_f64(k), to_f64(v), g.double().cpu().numpy(),
                                  dout.double().cpu().numpy(), cfg.block, cfg.topn, cfg.window,
                                  idx=sel.cpu().numpy())
    out = dict(dq=dq, dk=dk, dv=dv, dgates=dg)
    errs = {}
    for name, t in out.items():
        got = t.double().cpu().numpy()
        want = ref[name]
        assert np.all(np.isfinite(got)), name
        scale = float(np.abs(want).max())
        rel_l2 = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        max_rel = float(np.abs(got - want).max()) / scale
        errs[name] = (rel_l2, max_rel)
        log(f"{cfg.name} {name}: rel-L2 {rel_l2:.3e}, max-abs/max {max_rel:.3e} (max {scale:.3e})")
    for name, (rel_l2, max_rel) in errs.items():
        assert rel_l2 <= REL_L2, (name, rel_l2)
        assert max_rel <= MAX_REL, (name, max_rel)


def test_backward_ns32_two_heads():
    # N = 12288, block 64 (m = 192), top-16, window 256, d = 64
    _run(BSAConfig("ns32-bwd", 32, 1, 2, 64, 64, 16, 256, "iid", 32))


def test_backward_correlated_field_head_dim_32():
    _run(BSAConfig("ns32-d32", 32, 1, 1, 32, 64, 8, 100, "fourier", 33))


def _signed_gates(g):
    """Gates of either sign, with exact zeros and negative zeros: the interface
    takes any float32 gates, while the kernels fold each fine gate's sign into
    that branch's bf16 dO and its magnitude into the exponent of P|g|."""
    gen = torch.Generator(device=g.device).manual_seed(77)
    s = torch.randn(g.shape, generator=gen, device=g.device, dtype=torch.float32)
    s[..., 0::7, :] = 0.0
    s[..., 3::11, :] = -0.0
    return s


@pytest.mark.parametrize("use_saved", [False, True], ids=["recompute", "saved-state"])
def test_backward_signed_and_zero_gates(use_saved):
    _run(BSAConfig("ns32-signed", 32, 1, 2, 64, 64, 16, 256, "fourier", 38), gates=_signed_gates, use_saved=use_saved)


def test_backward_block_256():
    # N = 49152, block 256 (m = 192, four 64-query chunks per block), top-4
    _run(BSAConfig("ns64-b256", 64, 1, 1, 64, 256, 4, 300, "fourier", 34))


def _saved_views(saved: torch.Tensor, cfg: BSAConfig):
    """(o [S][N][2][d], lse [S][N][2]) from the training forward's state (layout of
    mosaic_bsa_saved_bytes: float32 branch outputs, then float32 log2-sum-exps, 256-byte sections)."""
    s, n, d = cfg.batch * cfg.heads, cfg.n_tokens, cfg.head_dim
    o_bytes = s * n * 2 * d * 4
    o = saved[:o_bytes].view(torch.float32).view(s, n, 2, d)
    lse_off = (o_bytes + 255) // 256 * 256
    lse = saved[lse_off:lse_off + s * n * 2 * 4].view(torch.float32).view(s, n, 2)
    return o, lse


@pytest.mark.parametrize("cfg", [
    BSAConfig("ns32-train", 32, 1, 2, 64, 64, 16, 256, "iid", 35),
    BSAConfig("ns64-b256-train", 64, 1, 1, 64, 256, 4, 300, "fourier", 36),
    BSAConfig("ns32-d32-train", 32, 1, 1, 32, 64, 8, 100, "fourier", 37),
], ids=lambda c: c.name)
def test_training_forward_state_and_backward(cfg):
    dev = "cuda"
    q, k, v, g = make_inputs(cfg, device=dev)
    out0, sel0 = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    out, sel, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    # the same selection; the same outputs up to float32 rounding of the gated sum
    assert torch.equal(sel, sel0)
    diff = float((out - out0).abs().max())
    log(f"{cfg.name} training forward vs forward: max-abs {diff:.3e}")
    assert diff <= 1e-6 * float(out0.abs().max())

    # the saved branch outputs and log2-sum-exps against the oracle, slice 0
    o, lse = _saved_views(saved, cfg)
    q0, k0, v0 = (to_f64(x)[0, 0] for x in (q, k, v))
    idx = sel[0, 0].cpu().numpy()
    o_fg = oracle.fine_selected_branch(q0, k0, v0, idx, cfg.block)
    o_l = oracle.local_branch(q0, k0, v0, cfg.window)
    for br, want in ((0, o_fg), (1, o_l)):
        got = o[0, :, br].double().cpu().numpy()
        err = float(np.abs(got - want).max())
        log(f"{cfg.name} saved o[{br}] max-abs {err:.3e}")
        assert err <= 1e-2
    # log2-sum-exp of q_t.k_u log2(e)/sqrt(d) over each branch's keys, for sampled queries
    d = cfg.head_dim
    rng = np.random.default_rng(cfg.seed)
    ts = rng.choice(cfg.n_tokens, size=64, replace=False)
    lo = np.maximum(ts - cfg.window // 2, 0)
    hi = np.minimum(ts + (cfg.window + 1) // 2, cfg.n_tokens)
    for j, t in enumerate(ts):
        blocks = idx[t // cfg.block]
        keys = (blocks[:, None] * cfg.block + np.arange(cfg.block)).ravel()
        for br, ks in ((0, keys), (1, np.arange(lo[j], hi[j]))):
            sc = k0[ks] @ q0[t] / np.sqrt(d)
            want = (sc.max() + np.log(np.exp(sc - sc.max()).sum())) / np.log(2.0)
            assert abs(float(lse[0, t, br]) - want) <= 2e-2 + 1e-3 * abs(want), (t, br)

    # backward from the saved state against the float64 oracle
    gen = torch.Generator(device=dev).manual_seed(2000 + cfg.seed)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32)
    dq, dk, dv, dg = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                              saved=saved)
    torch.cuda.synchronize()
    ref = oracle.bsa_backward_ref(to_f64(q), to_f64(k), to_f64(v), g.double().cpu().numpy(),
                                  dout.double().cpu().numpy(), cfg.block, cfg.topn, cfg.window,
                                  idx=sel.cpu().numpy())
    for name, t in dict(dq=dq, dk=dk, dv=dv, dgates=dg).items():
        got = t.double().cpu().numpy()
        want = ref[name]
        assert np.all(np.isfinite(got)), name
        rel_l2 = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        max_rel = float(np.abs(got - want).max()) / float(np.abs(want).max())
        log(f"{cfg.name} saved-state {name}: rel-L2 {rel_l2:.3e}, max-abs/max {max_rel:.3e}")
        assert rel_l2 <= REL_L2, (name, rel_l2)
        assert max_rel <= MAX_REL, (name, max_rel)


def _slice_backward_samples(q, k, v, g, do, sel, block, window, ts, key_blocks):
    """Oracle gradients of one slice at sampled query tokens (dq, dgates) and
    sampled key blocks (dk, dv), assembled from the oracle's per-branch
    pieces: ``attention_backward`` on each affected query's own key set, and
    ``compressed_backward`` on the whole pooled slice (selection fixed)."""
    n_tok, d = q.shape
    m = n_tok // block
    within = np.arange(block)
    qbar, kbar, vbar = (oracle.pool_mean(x, block) for x in (q, k, v))
    _, _, o_cg = oracle.compressed_branch(qbar, kbar, vbar)
    do_cg = (g[:, 0:1] * do).reshape(m, block, d).sum(axis=1)
    dqb, dkb, dvb = oracle.compressed_backward(qbar, kbar, vbar, do_cg)

    def sel_keys(i):
        return (np.asarray(sel[i], dtype=np.int64)[:, None] * block + within).ravel()

    def row(t, keys, gi):
        p = oracle.softmax_rows((q[t] @ k[keys].T / np.sqrt(d))[None])
        gq, gk, gv = oracle.attention_backward(q[t:t + 1], k[keys], v[keys], p, (g[t, gi] * do[t])[None])
        return p[0], gq[0], gk, gv

    dq, dg = [], []
    for t in ts:
        i = t // block
        ks = sel_keys(i)
        p_fg, gq_fg, _, _ = row(t, ks, 1)
        lo, hi = oracle.local_window_bounds(t, window, n_tok)
        kl = np.arange(int(lo), int(hi))
        p_l, gq_l, _, _ = row(t, kl, 2)
        dq.append(gq_fg + gq_l + dqb[i] / block)
        dg.append([do[t] @ o_cg[i], do[t] @ (p_fg @ v[ks]), do[t] @ (p_l @ v[kl])])

    dk, dv = [], []
    lo_off, hi_off = window // 2, window - window // 2
    for j in key_blocks:
        gk_j, gv_j = np.zeros((block, d)), np.zeros((block, d))
        for i in np.nonzero(np.any(np.asarray(sel) == j, axis=1))[0]:   # query blocks that chose block j
            rows = slice(i * block, (i + 1) * block)
            ks = sel_keys(i)
            p = oracle.softmax_rows(q[rows] @ k[ks].T / np.sqrt(d))
            _, gk, gv = oracle.attention_backward(q[rows], k[ks], v[ks], p, g[rows, 1:2] * do[rows])
            pos = np.nonzero(ks // block == j)[0]
            gk_j += gk[pos]
            gv_j += gv[pos]
        u0 = j * block
        for t in range(max(0, u0 - hi_off + 1), min(n_tok, u0 + block + lo_off)):   # queries whose window reaches the block
            lo, hi = oracle.local_window_bounds(t, window, n_tok)
            a, b = max(int(lo), u0), min(int(hi), u0 + block)
            if a >= b:
                continue
            _, _, gk, gv = row(t, np.arange(int(lo), int(hi)), 2)
            gk_j[a - u0:b - u0] += gk[a - int(lo):b - int(lo)]
            gv_j[a - u0:b - u0] += gv[a - int(lo):b - int(lo)]
        dk.append(gk_j + dkb[j] / block)
        dv.append(gv_j + dvb[j] / block)
    return np.array(dq), np.array(dg), np.concatenate(dk), np.concatenate(dv)


def test_backward_full_size_sampled():
    """The ns128 bench workload (24 members x 8 heads, block 64, top-16, window
    512) in the launch configuration bench.py times (training forward, then the
    backward from its state): two slices checked at 48 sampled query tokens
    (dq, dgates) and at the most and least selected key blocks plus one
    random one (dk, dv)."""
    cfg = BSAConfig("ns128", 128, 24, 8, 64, 64, 16, 512, "fourier", 128)
    dev = "cuda"
    q, k, v, g = make_inputs(cfg, device=dev)
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 7)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32)
    _, sel, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    dq, dk, dv, dg = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                              saved=saved)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for bi, hi in ((5, 3), (17, 6)):
        s_ = sel[bi, hi].cpu().numpy()
        counts = np.bincount(s_.ravel(), minlength=cfg.n_blocks)
        kb = [int(np.argmax(counts)), int(np.argmin(counts)), int(rng.integers(0, cfg.n_blocks))]
        ts = np.sort(rng.choice(cfg.n_tokens, 48, replace=False))
        ts[:2] = (0, cfg.n_tokens - 1)                     # the clipped windows at both ends
        args = [to_f64(x[bi, hi]) for x in (q, k, v, g, dout)]
        rq, rg, rk, rv = _slice_backward_samples(*args, s_, cfg.block, cfg.window, ts, kb)
        keys = np.concatenate([np.arange(j * cfg.block, (j + 1) * cfg.block) for j in kb])
        pairs = (("dq", to_f64(dq[bi, hi])[ts], rq), ("dgates", to_f64(dg[bi, hi])[ts], rg),
                 ("dk", to_f64(dk[bi, hi])[keys], rk), ("dv", to_f64(dv[bi, hi])[keys], rv))
        for name, got, want in pairs:
            rel_l2 = float(np.linalg.norm(got - want) / np.linalg.norm(want))
            max_rel = float(np.abs(got - want).max()) / float(np.abs(want).max())
            log(f"ns128 slice ({bi},{hi}) {name}: rel-L2 {rel_l2:.3e}, max-abs/max {max_rel:.3e} "
                f"(key blocks {kb}, selected by {counts[kb].tolist()} query blocks)")
            assert rel_l2 <= REL_L2, (name, rel_l2)
            assert max_rel <= MAX_REL, (name, max_rel)
