"""GPU parity of the encoder layer (input projection, BSA, output projection)
against the float64 oracle ``oracle.layer``, through the C ABI.

Rounding: the GPU accumulates the projections in float32 and rounds q, k, v,
the merged attention output and y to bf16 once; the oracle rounds the exact
float64 sums.  Both round to nearest even, so an element differs only when
the float32 sum and the exact sum straddle a rounding boundary: by one bf16
ulp (2^-8 relative at most), in a small fraction of elements.  The stage
tests check exactly that.  The whole layer is checked with the oracle's
selection forced to the GPU's (the one-ulp input differences move the
compressed logits by far less than the selection gaps checked here), with
the tolerance of the attention output (rel-L2 <= 5e-3, max-abs <= 1e-2 of
the attention) carried through the output projection.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import BSAConfig, _lib, make_inputs, make_layer_inputs
from spherical_block_sparse_amd.synth import to_f64

from parity import check_indices, log, selection_ref

pytestmark = pytest.mark.gpu


def _ulp_check(name, got, want, absum, k, min_exact=0.99):
    """got within one bf16 ulp plus the float32 summation bound of want, and
    equal in most places.  A float32 sum of k terms errs by at most
    k * 2^-24 * (sum of their magnitudes) = k * 2^-24 * absum; rounding that
    sum to bf16 adds at most one ulp of the result."""
    got, want = np.asarray(got), np.asarray(want)
    mag = np.maximum(np.abs(want), np.abs(got))
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
    allowed = ulp + k * 2.0 ** -24 * np.asarray(absum)
    diff = np.abs(got - want)
    exact = float(np.mean(diff == 0))
    worst = float(np.max(diff / allowed))
    log(f"{name}: exact {exact:.5f}, worst {worst:.3f} of the bound")
    assert worst <= 1.0, name
    assert exact >= min_exact, name


def _split(z, heads, head_dim):
    b, n, _ = z.shape
    return z.reshape(b, n, heads, head_dim).transpose(0, 2, 1, 3)


LAYER_CASES = [
    # (config, channels): ragged token and feature tiles, head_dim 32 and 64
    (BSAConfig("ns4-layer", 4, 1, 2, 32, 16, 2, 24, "iid", 41), 64),
    (BSAConfig("ns8-layer", 8, 2, 2, 64, 16, 4, 32, "iid", 42), 128),
    (BSAConfig("ns16-layer", 16, 1, 4, 64, 64, 8, 128, "fourier", 43), 256),
]


@pytest.mark.parametrize("cfg,channels", LAYER_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_layer_input_projection(cfg, channels):
    x, w_in, _ = make_layer_inputs(cfg, channels, device="cuda")
    q, k, v, g = _lib.mosaic_bsa_layer_in(x, w_in[0], cfg.heads, cfg.head_dim, cfg.nside)
    torch.cuda.synchronize()
    xf, wf = to_f64(x), to_f64(w_in[0])
    rq, rk, rv, rg = oracle.layer_in_ref(xf, wf, cfg.heads, cfg.head_dim)
    hd = cfg.heads * cfg.head_dim
    absum = np.abs(xf) @ np.abs(wf).T
    for i, (name, got, want) in enumerate((("q", q, rq), ("k", k, rk), ("v", v, rv))):
        _ulp_check(f"{cfg.name} {name}", to_f64(got), want,
                   _split(absum[..., i * hd:(i + 1) * hd], cfg.heads, cfg.head_dim), channels)
    err = float(np.abs(to_f64(g) - rg).max())
    log(f"{cfg.name} gates max-abs {err:.2e}")
    assert err <= 2e-6


@pytest.mark.parametrize("cfg,channels", LAYER_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_layer_output_projection(cfg, channels):
    x, _, w_out = make_layer_inputs(cfg, channels, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    attn = torch.randn((cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim), generator=gen, device="cuda")
    y = _lib.mosaic_bsa_layer_out(attn, w_out[0], x, cfg.nside)
    torch.cuda.synchronize()
    a, wo, xf = to_f64(attn), to_f64(w_out[0]), to_f64(x)
    want = oracle.layer_out_ref(a, wo, xf)
    b, h, n, d = a.shape
    absum = np.abs(xf) + np.abs(a.transpose(0, 2, 1, 3).reshape(b, n, h * d)) @ np.abs(wo).T
    _ulp_check(f"{cfg.name} y", to_f64(y), want, absum, h * d + 1)


@pytest.mark.parametrize("cfg,channels", LAYER_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_layer_output_projection_merged(cfg, channels):
    """The merged-layout entry point (the layer's own GEMM) against the
    oracle on the same bf16 attention values, and in place (y = x)."""
    x, _, w_out = make_layer_inputs(cfg, channels, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 1)
    b, h, n, d = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim
    attn = torch.randn((b, h, n, d), generator=gen, device="cuda").to(torch.bfloat16)
    merged = attn.permute(0, 2, 1, 3).contiguous().view(b, n, h * d)
    y = _lib.mosaic_bsa_layer_out_merged(merged, w_out[0], x, cfg.nside, h)
    y_in_place = x.clone()
    _lib.mosaic_bsa_layer_out_merged(merged, w_out[0], y_in_place, cfg.nside, h, y=y_in_place)
    torch.cuda.synchronize()
    assert torch.equal(y, y_in_place)
    a, wo, xf = to_f64(attn), to_f64(w_out[0]), to_f64(x)
    want = oracle.layer_out_ref(a, wo, xf)
    absum = np.abs(xf) + np.abs(a.transpose(0, 2, 1, 3).reshape(b, n, h * d)) @ np.abs(wo).T
    _ulp_check(f"{cfg.name} y (merged)", to_f64(y), want, absum, h * d + 1)
    # the float32 stage entry point on the same (bf16-valued) attention output agrees
    y32 = _lib.mosaic_bsa_layer_out(attn.float(), w_out[0], x, cfg.nside)
    torch.cuda.synchronize()
    assert float((y.float() == y32.float()).float().mean()) >= 0.999


@pytest.mark.parametrize("cfg,channels", LAYER_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_layer_forward(cfg, channels):
    x, w_in, w_out = make_layer_inputs(cfg, channels, device="cuda")
    y, sel = _lib.mosaic_bsa_layer_forward(x, w_in[0], w_out[0], cfg.heads, cfg.head_dim, cfg.nside, cfg.block,
                                           cfg.topn, cfg.window)
    # the layer equals its stages run one after another: the same selection;
    # y up to the rounding of the attention output, which the layer takes
    # straight to bf16 inside the fine kernel
    q, k, v, g = _lib.mosaic_bsa_layer_in(x, w_in[0], cfg.heads, cfg.head_dim, cfg.nside)
    attn, sel2 = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    y2 = _lib.mosaic_bsa_layer_out(attn, w_out[0], x, cfg.nside)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    same = float((y == y2).float().mean())
    log(f"{cfg.name} layer vs stages: {same:.5f} of y equal")
    assert same >= 0.999
    assert float((y.float() - y2.float()).abs().max()) <= 2.0 ** -7 * float(y2.float().abs().max())

    ref = oracle.layer_ref(to_f64(x), to_f64(w_in[0]), to_f64(w_out[0]), cfg.heads, cfg.head_dim, cfg.block,
                           cfg.topn, cfg.window, idx=sel.cpu().numpy())
    own = oracle.layer_ref(to_f64(x), to_f64(w_in[0]), to_f64(w_out[0]), cfg.heads, cfg.head_dim, cfg.block,
                           cfg.topn, cfg.window)
    # on the GPU's own bf16 q, k, v the selection is the oracle's bit for bit (near ties of
    # 1e-6 aside), as in the attention's parity tests
    near = 0
    for bi in range(cfg.batch):
        for hh in range(cfg.heads):
            r = selection_ref(to_f64(q[bi, hh]), to_f64(k[bi, hh]), to_f64(v[bi, hh]), cfg.block, cfg.topn)
            near += check_indices(sel[bi, hh].cpu().numpy(), r, cfg.topn)["near_ties"]
    log(f"{cfg.name} selection on the GPU's q, k, v: bit-exact except {near} near-tie rows")
    # against the oracle's own projections q, k, v may differ by one bf16 ulp, so only rows
    # whose gap no such change can close are compared
    clear = own["gap"] > 1e-3          # rows whose selection no one-ulp input change can flip
    agree = np.all(own["idx"] == sel.cpu().numpy(), axis=-1)
    log(f"{cfg.name} selection: {int(np.sum(agree & clear))} of {int(np.sum(clear))} clear rows agree")
    assert np.all(agree[clear])
    got, want = to_f64(y), ref["y"]
    delta = got - want
    # the attention's own tolerance, through w_out: |w_out| rows have norm ~1
    rel = float(np.linalg.norm(delta) / np.linalg.norm(want - to_f64(x)))
    log(f"{cfg.name} y: rel-L2 of the update {rel:.2e}, max-abs {float(np.abs(delta).max()):.2e}")
    assert rel <= 1e-2
    assert float(np.abs(delta).max()) <= 2e-2 * float(np.abs(want).max())


def test_layer_full_size_sampled_tokens():
    """The ns128 bench workload (24 members x 8 heads x 64, 512 channels): the
    two projections checked on 256 sampled tokens against the oracle's
    per-token formulas."""
    cfg = BSAConfig("ns128", 128, 24, 8, 64, 64, 16, 512, "fourier", 128)
    c = 512
    x, w_in, w_out = make_layer_inputs(cfg, c, device="cuda")
    q, k, v, g = _lib.mosaic_bsa_layer_in(x, w_in[0], cfg.heads, cfg.head_dim, cfg.nside)
    gen = torch.Generator(device="cuda").manual_seed(5)
    attn = torch.randn((cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim), generator=gen, device="cuda")
    y = _lib.mosaic_bsa_layer_out(attn, w_out[0], x, cfg.nside)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    bs = rng.integers(0, cfg.batch, 256)
    ts = rng.integers(0, cfg.n_tokens, 256)
    xs = to_f64(x[bs, ts])[:, None, :]                              # [256, 1, C] as 256 one-token batches
    wi, wo = to_f64(w_in[0]), to_f64(w_out[0])
    rq, rk, rv, rg = oracle.layer_in_ref(xs, wi, cfg.heads, cfg.head_dim)
    hd = cfg.heads * cfg.head_dim
    absum = np.abs(xs) @ np.abs(wi).T
    bt = (torch.from_numpy(bs).cuda(), slice(None), torch.from_numpy(ts).cuda())
    _ulp_check("ns128 q sampled", to_f64(q[bt])[:, :, None, :], rq, _split(absum[..., :hd], cfg.heads, cfg.head_dim), c)
    _ulp_check("ns128 v sampled", to_f64(v[bt])[:, :, None, :], rv,
               _split(absum[..., 2 * hd:3 * hd], cfg.heads, cfg.head_dim), c)
    assert float(np.abs(to_f64(g[bt])[:, :, None, :] - rg).max()) <= 2e-6
    a = to_f64(attn[bt])[:, :, None, :]
    ry = oracle.layer_out_ref(a, wo, xs)
    absum_y = np.abs(xs) + np.abs(a.transpose(0, 2, 1, 3).reshape(256, 1, hd)) @ np.abs(wo).T
    _ulp_check("ns128 y sampled", to_f64(y[bs, ts])[:, None, :], ry, absum_y, hd + 1)
