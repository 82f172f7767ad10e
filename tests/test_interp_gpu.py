"""GPU parity of the lat-lon -> HEALPix cross-attention interpolation
(mosaic_interp_attention) against the float64 oracle ``oracle.interp``.

Error budget of the kernel: kappa_j = W_q^T k_j / sqrt(d) is a float32 sum
of d exact products (relative error ~d * 2^-24), the 16 scores and their
softmax are float32 (fast exp, a few ulp), and the output is a float32 sum of
16 products of the weights with exact bf16 values.  Each output element is
then within ~1e-6 of the oracle relative to the largest |v| of its
neighbourhood; the test allows 2e-5 of the largest |v| overall."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import _lib
from spherical_block_sparse_amd.synth import make_interp_inputs, to_f64

from parity import log

pytestmark = pytest.mark.gpu


def _check(name, got, want, vmax):
    err = float(np.abs(got - want).max())
    log(f"{name}: max-abs {err:.2e} (max |v| {vmax:.2f})")
    assert err <= 2e-5 * vmax


@pytest.mark.parametrize("nside,n_lat,n_lon,slices,d", [(8, 37, 72, 2, 64), (32, 181, 360, 2, 32), (16, 91, 180, 3, 128)])
def test_interp_matches_oracle(nside, n_lat, n_lon, slices, d):
    k, v, w_q, nbr, rel = make_interp_inputs(nside, n_lat, n_lon, slices, d=d, device="cuda", seed=nside)
    out = _lib.mosaic_interp_attention(k, v, w_q, nbr, rel)
    torch.cuda.synchronize()
    want = oracle.interp_attention_ref(to_f64(k), to_f64(v), to_f64(w_q), nbr.cpu().numpy(), to_f64(rel))
    _check(f"interp ns{nside} {n_lat}x{n_lon} d{d}", to_f64(out), want, float(v.float().abs().max()))


def test_interp_fewer_neighbours():
    # the first 9 stencil points only (n_nbr < 16 leaves lanes idle)
    k, v, w_q, nbr, rel = make_interp_inputs(8, 37, 72, 2, device="cuda", seed=3)
    nbr9, rel9 = nbr[:, :9].contiguous(), rel[:, :9].contiguous()
    out = _lib.mosaic_interp_attention(k, v, w_q, nbr9, rel9)
    torch.cuda.synchronize()
    want = oracle.interp_attention_ref(to_f64(k), to_f64(v), to_f64(w_q), nbr9.cpu().numpy(), to_f64(rel9))
    _check("interp 9 neighbours", to_f64(out), want, float(v.float().abs().max()))


def test_interp_full_size_sampled():
    """The 0.25-degree grid (721 x 1440) onto Nside 256 for 32 slices (2
    members x 16 heads), 512 sampled (slice, target) outputs."""
    k, v, w_q, nbr, rel = make_interp_inputs(256, 721, 1440, 32, device="cuda", seed=256)
    out = _lib.mosaic_interp_attention(k, v, w_q, nbr, rel)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    ss, ts = rng.integers(0, 32, 512), rng.integers(0, nbr.shape[0], 512)
    nb, rl, wq = nbr.cpu().numpy(), to_f64(rel), to_f64(w_q)
    vmax = float(v.float().abs().max())
    worst = 0.0
    for s in np.unique(ss):
        sel = ts[ss == s]
        want = oracle.interp_attention(to_f64(k[s]), to_f64(v[s]), wq, nb[sel], rl[sel])
        got = to_f64(out[s, torch.from_numpy(sel).cuda()])
        worst = max(worst, float(np.abs(got - want).max()))
    log(f"interp full size sampled: max-abs {worst:.2e} (max |v| {vmax:.2f})")
    assert worst <= 2e-5 * vmax
