"""Pins of the float64 interpolation oracle (``oracle.interp``): closed forms
(zero query weights give the neighbourhood mean, one neighbour gives its
value), torch's float64 scaled_dot_product_attention where every neighbour
sits at the same relative position (one query per target), invariance to
the neighbour order, and the stencil's geometry."""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import interp_attention
from spherical_block_sparse_amd.synth import latlon_stencil, latlon_vectors, pix2vec_nest


def _rand(seed, n_src=200, n_dst=50, K=16, d=8, dv=6):
    r = np.random.default_rng(seed)
    return (r.standard_normal((n_src, d)), r.standard_normal((n_src, dv)), r.standard_normal((d, 3)),
            r.integers(0, n_src, (n_dst, K)), r.standard_normal((n_dst, K, 3)))


def test_zero_query_weights_give_the_neighbourhood_mean():
    k, v, w, nbr, rel = _rand(0)
    np.testing.assert_allclose(interp_attention(k, v, 0 * w, nbr, rel), v[nbr].mean(axis=1), rtol=1e-13)


def test_single_neighbour_returns_its_value():
    k, v, w, nbr, rel = _rand(1, K=1)
    np.testing.assert_array_equal(interp_attention(k, v, w, nbr, rel), v[nbr[:, 0]])


def test_equal_relative_positions_match_library_attention():
    k, v, w, nbr, rel = _rand(2)
    rel[:] = rel[:, :1, :]                               # every neighbour at the target's first offset
    q = rel[:, 0, :] @ w.T                               # one query per target
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, None, :], torch.from_numpy(k[nbr])[:, None], torch.from_numpy(v[nbr])[:, None]
    )[:, 0, 0].numpy()
    np.testing.assert_allclose(interp_attention(k, v, w, nbr, rel), want, rtol=1e-12, atol=1e-14)


def test_neighbour_order_does_not_matter():
    k, v, w, nbr, rel = _rand(3)
    perm = np.random.default_rng(4).permutation(nbr.shape[1])
    np.testing.assert_allclose(interp_attention(k, v, w, nbr[:, perm], rel[:, perm]),
                               interp_attention(k, v, w, nbr, rel), rtol=1e-13)


def test_stencil_surrounds_each_target():
    nside, n_lat, n_lon = 8, 37, 72
    nbr, rel = latlon_stencil(nside, n_lat, n_lon)
    u = pix2vec_nest(nside)
    src = latlon_vectors(n_lat, n_lon)
    spacing = math.radians(180.0 / (n_lat - 1))
    np.testing.assert_allclose(rel, (src[nbr] - u[:, None, :]) / spacing, rtol=1e-5, atol=1e-6)
    # the nearest grid point of every target is in its stencil (brute force over the grid)
    nearest = np.argmax(u @ src.T, axis=1)
    near_ok = [(nearest[i] in set(nbr[i])) or np.isclose(u[i] @ src[nearest[i]], (u[i] @ src[nbr[i]].T).max())
               for i in range(len(u))]
    assert all(near_ok)
    # every stencil point lies within ~2.2 grid spacings of the target (away from the pole rows)
    dist = np.linalg.norm(rel, axis=-1)
    assert np.all(dist[np.abs(u[:, 2]) < 0.9] < 3.2)
