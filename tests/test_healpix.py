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
