"""Float64 reference of the lat-lon -> HEALPix cross-attention interpolation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy float64.

Source: papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED: each
HEALPix target point i takes the relative positions p_ij of its neighbouring
source points j as queries and the source features as keys and values,
o_i = sum_{j in N_i} softmax_j(q_ij^T k_j / sqrt(d)) v_j.  Readings taken
(the pages fix neither):

  i1  q_ij = W_q p_ij, one linear map (d x 3) of the relative position
      p_ij = (u_j - u_i) / spacing (unit vectors, grid spacing in radians).
  i2  N_i is the 4 x 4 block of lat-lon grid points around the target's
      centre (rows clamped at the poles, so polar stencils repeat a row;
      columns wrap in longitude); k_j and v_j are given per source point.
  i3  one softmax over the listed neighbours; a repeated neighbour counts
      once per listing.
"""

from __future__ import annotations

import numpy as np

from .bsa import _f64, softmax_rows


def interp_attention(k, v, w_q, nbr, rel) -> np.ndarray:
    """One slice: k [n_src, d], v [n_src, dv], w_q [d, 3], nbr [n_dst, K]
    source indices, rel [n_dst, K, 3] relative positions -> o [n_dst, dv]."""
    k, v, w_q, rel = _f64(k), _f64(v), _f64(w_q), _f64(rel)
    nbr = np.asarray(nbr, dtype=np.int64)
    d = k.shape[1]
    q = rel @ w_q.T                                   # q_ij, [n_dst, K, d]
    s = np.sum(q * k[nbr], axis=-1) / np.sqrt(d)      # [n_dst, K]
    p = softmax_rows(s)
    return np.einsum("ik,ikc->ic", p, v[nbr])


def interp_attention_ref(k, v, w_q, nbr, rel) -> np.ndarray:
    """``interp_attention`` over slices: k [S, n_src, d], v [S, n_src, dv]."""
    k = np.asarray(k)
    return np.stack([interp_attention(k[s], v[s], w_q, nbr, rel) for s in range(k.shape[0])])
