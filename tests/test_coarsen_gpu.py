"""GPU parity of HEALPix NESTED coarsening (mosaic_healpix_coarsen) against
the float64 oracle ``oracle.healpix.coarsen`` (mean of each coarse pixel's
descendants, children rule applied level by level).

The kernel sums in float64 and rounds the mean once to float32, so each
element is within one float32 rounding (2^-24 relative) of the oracle plus
the float64 summation error (negligible here)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import BSAConfig, _lib, make_layer_inputs
from spherical_block_sparse_amd.synth import to_f64

from parity import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nside,channels,levels", [(8, 8, 1), (8, 64, 3), (32, 64, 1), (32, 24, 2), (16, 512, 4)])
def test_coarsen_matches_oracle(nside, channels, levels):
    cfg = BSAConfig(f"ns{nside}-coarsen", nside, 2, 1, 64, 16, 1, 1, "fourier", 50 + nside)
    x, _, _ = make_layer_inputs(cfg, channels, device="cuda")
    y = _lib.mosaic_healpix_coarsen(x, nside, levels)
    torch.cuda.synchronize()
    want = oracle.coarsen(to_f64(x), nside, levels)
    got = to_f64(y)
    err = np.abs(got - want)
    bound = 2.0 ** -24 * np.abs(want) * 1.000001 + 1e-30
    log(f"coarsen ns{nside} C{channels} L{levels}: worst {float(np.max(err / bound)):.3f} of one float32 rounding")
    assert np.all(err <= bound)


def test_coarsen_full_size_sampled():
    # the ns128 bench mesh at 512 channels, two levels (Nside 128 -> 32), 64 sampled coarse pixels
    cfg = BSAConfig("ns128-coarsen", 128, 4, 1, 64, 16, 1, 1, "fourier", 128)
    x, _, _ = make_layer_inputs(cfg, 512, device="cuda")
    y = _lib.mosaic_healpix_coarsen(x, 128, 2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for b, p in zip(rng.integers(0, 4, 64), rng.integers(0, 12 * 32 * 32, 64)):
        kids = oracle.descendants(int(p), 2)
        want = to_f64(x[b, kids]).mean(axis=0)
        got = to_f64(y[b, p])
        assert np.all(np.abs(got - want) <= 2.0 ** -24 * np.abs(want) * 1.000001 + 1e-30)
