"""Seeded random shapes through the training forward and the backward, every
gradient element against the float64 oracle backward.

The backward takes blocks of at least 64 tokens, top-n up to 64 and
m = N/block a multiple of 64.  A fixed seed draws shapes inside that domain
that the hand-picked cases do not: Nside 32 or 64, blocks of 64 or 256, any
top-n from 1 to min(m, 64), windows from 1 to past the sphere (at Nside 32;
up to 2000 at Nside 64), head_dim 32
or 64, one or two slices, i.i.d. or correlated fields, and gates of either
sign with exact zeros in a third of the cases.  Each case runs both the
backward that recomputes the forward's state and the one from the training
forward's saved state, and prints its shape before it touches the GPU.
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
N_CASES = 10


def random_backward_shapes(seed: int = 20261205, count: int = N_CASES) -> list[tuple[BSAConfig, bool]]:
    """Valid backward shapes (and whether the gates are signed) from a fixed seed; host only."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        nside, block = [(32, 64), (64, 64), (64, 256)][int(rng.choice(3, p=[0.5, 0.2, 0.3]))]
        n_tok = 12 * nside * nside
        m = n_tok // block
        topn = int(rng.integers(1, min(m, 64) + 1))
        # windows past the sphere only at Nside 32 (the oracle's local branch is then dense)
        wide = int(rng.integers(n_tok, 2 * n_tok + 8)) if nside == 32 else int(rng.integers(700, 2000))
        window = int(rng.choice([1, int(rng.integers(2, 64)), int(rng.integers(64, 700)), wide]))
        head_dim = int(rng.choice([32, 64]))
        heads = int(rng.integers(1, 3)) if nside == 32 else 1
        field = "fourier" if rng.random() < 0.5 else "iid"
        signed = bool(rng.random() < 1 / 3)
        name = f"rb{i:02d}-s{nside}-b{block}-n{topn}-w{window}-d{head_dim}{'-signed' if signed else ''}"
        out.append((BSAConfig(name, nside, 1, heads, head_dim, block, topn, window, field, 6000 + i), signed))
    # and the corner the draw may miss: the largest top-n with a window past the sphere
    out.append((BSAConfig("rb-s32-b64-n64-wide-d64-signed", 32, 1, 2, 64, 64, 64, 2 * 12 * 32 * 32 + 1, "fourier",
                          6999), True))
    return out


CASES = random_backward_shapes()


def _signed(g, seed):
    gen = torch.Generator(device=g.device).manual_seed(seed)
    s = torch.randn(g.shape, generator=gen, device=g.device, dtype=torch.float32)
    s[..., 0::5, :] = 0.0
    s[..., 2::9, :] = -0.0
    return s


@pytest.mark.parametrize("cfg,signed", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_random_shape_backward(cfg, signed):
    log(f"[case] {cfg.name}: nside={cfg.nside} H={cfg.heads} d={cfg.head_dim} block={cfg.block} topn={cfg.topn} "
        f"W={cfg.window} field={cfg.field} signed={signed} seed={cfg.seed}")
    dev = "cuda"
    q, k, v, g = make_inputs(cfg, device=dev)
    if signed:
        g = _signed(g, cfg.seed)
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 1)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32)
    _, sel, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    from_state = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                          saved=saved)
    recomputed = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    ref = oracle.bsa_backward_ref(to_f64(q), to_f64(k), to_f64(v), g.double().cpu().numpy(),
                                  dout.double().cpu().numpy(), cfg.block, cfg.topn, cfg.window,
                                  idx=sel.cpu().numpy())
    for how, grads in (("saved", from_state), ("recomputed", recomputed)):
        for name, t in zip(("dq", "dk", "dv", "dgates"), grads):
            got = t.double().cpu().numpy()
            want = ref[name]
            assert np.all(np.isfinite(got)), (how, name)
            scale = float(np.abs(want).max())
            rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
            max_rel = float(np.abs(got - want).max()) / max(scale, 1e-300)
            log(f"    {how} {name}: rel-L2 {rel_l2:.3e}, max-abs/max {max_rel:.3e}")
            assert rel_l2 <= REL_L2, (how, name, rel_l2)
            assert max_rel <= MAX_REL, (how, name, max_rel)
