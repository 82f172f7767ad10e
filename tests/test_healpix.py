"""HEALPix NESTED facts: the oracle's index helpers and the generator's pixel centres.

The index facts (N = 12*Nside^2, children 4p..4p+3) come from the
papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED.  The pixel-centre
geometry is textbook HEALPix (Gorski et al. 2005) and only shapes the
synthetic fields; it does not enter the BSA arithmetic.
"""

import os

import numpy as np
import pytest

from oracle import healpix
from spherical_block_sparse_amd.synth import pix2vec_nest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "healpix_centres.txt")


@pytest.mark.parametrize("nside", [1, 2, 4, 8, 32, 64, 128, 256])
def test_npix(nside):
    assert healpix.npix(nside) == 12 * nside * nside
    if nside <= 64:
        assert pix2vec_nest(nside).shape == (12 * nside * nside, 3)


def test_children_rule():
    for p in [0, 1, 5, 11, 47, 1000]:
        assert healpix.nest_children(p) == [4 * p, 4 * p + 1, 4 * p + 2, 4 * p + 3]
        for c in healpix.nest_children(p):
            assert healpix.nest_parent(c) == p


@pytest.mark.parametrize("levels", [1, 2, 3, 4])
def test_descendants_are_contiguous_blocks(levels):
    # block size B = 4^k: block i of the fine grid == coarse pixel i's descendants
    B = 4 ** levels
    for i in [0, 1, 7, 11, 30]:
        assert healpix.descendants(i, levels) == list(range(i * B, (i + 1) * B))


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            ns, p, zn, zd, fn, fd = map(int, line.split())
            rows.append((ns, p, zn / zd, np.pi * fn / fd))
    return rows


def test_pixel_centres_match_textbook_values():
    rows = _golden_rows()
    assert len(rows) == 16
    for ns, p, z, phi in rows:
        vec = pix2vec_nest(ns)[p]
        want = np.array([np.sqrt(1 - z * z) * np.cos(phi), np.sqrt(1 - z * z) * np.sin(phi), z])
        np.testing.assert_allclose(vec, want, atol=1e-14)


@pytest.mark.parametrize("nside", [1, 2, 4, 8, 16])
def test_pixel_centre_rings(nside):
    v = pix2vec_nest(nside)
    np.testing.assert_allclose(np.linalg.norm(v, axis=1), 1.0, atol=1e-14)
    z = np.round(v[:, 2], 12)
    zs, counts = np.unique(z, return_counts=True)
    assert zs.size == 4 * nside - 1
    counts = counts[::-1]                              # north to south
    for i in range(1, nside):                          # polar caps: ring i has 4i pixels
        assert counts[i - 1] == 4 * i
        assert counts[-i] == 4 * i
    assert np.all(counts[nside - 1:3 * nside] == 4 * nside)   # equatorial belt
    np.testing.assert_allclose(v.sum(axis=0), 0.0, atol=1e-9)  # symmetric tessellation


@pytest.mark.parametrize("nside", [1, 2, 4, 8, 16])
def test_children_lie_inside_parent(nside):
    """Each child's centre lies within one parent pixel size of the parent's
    centre, and the four children average (on the sphere) near the parent."""
    parent = pix2vec_nest(nside)
    child = pix2vec_nest(2 * nside).reshape(-1, 4, 3)
    size = np.sqrt(np.pi / 3.0) / nside                  # angular pixel size
    ang = np.arccos(np.clip(np.einsum("pcx,px->pc", child, parent), -1, 1))
    assert ang.max() < size
    mean = child.mean(axis=1)
    mean /= np.linalg.norm(mean, axis=1, keepdims=True)
    assert np.arccos(np.clip(np.einsum("px,px->p", mean, parent), -1, 1)).max() < 0.5 * size


def test_centres_distinct():
    v = pix2vec_nest(8)
    assert np.unique(np.round(v, 10), axis=0).shape[0] == v.shape[0]


def test_coarsen_pins():
    from oracle import coarsen, npix, pool_mean
    r = np.random.default_rng(7)
    nside = 8
    x = r.standard_normal((2, npix(nside), 5))
    # one level twice equals two levels at once (means of equal-size groups)
    np.testing.assert_allclose(coarsen(coarsen(x, nside, 1), nside // 2, 1), coarsen(x, nside, 2), rtol=1e-12, atol=1e-15)
    # the global mean is kept
    np.testing.assert_allclose(coarsen(x, nside, 3).mean(axis=1), x.mean(axis=1), rtol=1e-12)
    # a field constant on the coarse pixels comes back unchanged
    c = r.integers(-64, 64, (npix(nside // 4), 5)) / 8.0   # dyadic: the sums are exact
    np.testing.assert_array_equal(coarsen(np.repeat(c, 16, axis=0), nside, 2), c)
    # equals the BSA oracle's block mean with block 4^levels (reshape-mean, written separately)
    np.testing.assert_allclose(coarsen(x[0], nside, 2), pool_mean(x[0], 16), rtol=1e-12, atol=1e-15)
    # levels 0 is the identity
    np.testing.assert_array_equal(coarsen(x, nside, 0), x)


def test_ring_order_textbook_values():
    from spherical_block_sparse_amd.synth import nest_ring_order
    # at Nside 1 the two schemes number the 12 base pixels alike
    np.testing.assert_array_equal(nest_ring_order(1), np.arange(12))
    # Nside 2: the polar ring is the top corner (child 3) of base pixels 0..3,
    # the next ring alternates children 2 and 1; the south polar ring is child 0 of 8..11
    o = nest_ring_order(2)
    np.testing.assert_array_equal(o[:12], [3, 7, 11, 15, 2, 1, 6, 5, 10, 9, 14, 13])
    np.testing.assert_array_equal(o[-4:], [32, 36, 40, 44])
    for nside in (4, 16):
        o = nest_ring_order(nside)
        assert sorted(o.tolist()) == list(range(healpix.npix(nside)))
        v = pix2vec_nest(nside)[o]
        assert np.all(np.diff(v[:, 2]) <= 1e-12)              # north to south
        phi = np.mod(np.arctan2(v[:, 1], v[:, 0]), 2 * np.pi)
        same_ring = np.abs(np.diff(v[:, 2])) < 1e-12
        assert np.all(np.diff(phi)[same_ring] > 0)            # eastward inside a ring
