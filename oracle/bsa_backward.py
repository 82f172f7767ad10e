"""Float64 reference of the BSA backward pass, one (batch, head) slice at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy float64.

The forward followed is the one of ``oracle.bsa`` (papernotes.org ICML2026
notes, 关键设计 › "Mesh-aligned Block-Sparse Attention (BSA)"): pooled block
summaries, a compressed branch, a selected branch over the top-n key blocks of
each query block, a local window branch, and the gated sum
out_t = g_CG·o_CG[t // B] + g_FG·o_FG_t + g_L·o_L_t.  The pages give no
backward; the papernotes page says the model is trained end to end, so the
gradient of that forward with respect to q, k, v and the gates is what is
computed here.  Readings taken (the pages are silent on all of them):

  g1  the selected block indices are constants: top-n is piecewise constant,
      so its derivative is zero wherever it is defined.
  g2  gradients of the pooled means flow back uniformly: d x_t += d x̄_i / B
      for every token t of block i (derivative of the mean, reading c1).
  g3  the gates are inputs and receive dg_t = (dO_t·o_CG[t // B],
      dO_t·o_FG_t, dO_t·o_L_t).

Every softmax-attention branch o = P V, P = softmax_rows(q k^T / sqrt(d)) over
its own key set, has the standard gradient, written out in
``attention_backward``.
"""

from __future__ import annotations

import numpy as np

from .bsa import (
    _f64,
    _check_shape,
    compressed_branch,
    fine_selected_branch,
    local_branch,
    local_window_bounds,
    pool_mean,
    select_topn,
    softmax_rows,
)


def attention_backward(q, k, v, p, do):
    """Gradient of o = P V, P = softmax_rows(q k^T / sqrt(d)), given dO.

    p holds the probabilities of the forward (0 for excluded keys).  With
    dP = dO V^T and D_r = sum_u P_ru dP_ru (= dO_r · o_r), the logit gradient
    is dS = P ⊙ (dP - D); then dq = dS k / sqrt(d), dk = dS^T q / sqrt(d),
    dv = P^T dO.  Returns (dq, dk, dv)."""
    q, k, v, p, do = _f64(q), _f64(k), _f64(v), _f64(p), _f64(do)
    d = q.shape[1]
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=1, keepdims=True)
    ds = p * (dp - dsum)
    return ds @ k / np.sqrt(d), ds.T @ q / np.sqrt(d), dv


def pool_backward(dxbar, block: int) -> np.ndarray:
    """Reading g2: gradient of the block mean, spread over the block's tokens.
    dxbar [m, d] -> [m*block, d]."""
    return np.repeat(_f64(dxbar) / block, block, axis=0)


def compressed_backward(qbar, kbar, vbar, do_cg):
    """Gradient of the compressed branch o_CG = softmax(q̄ k̄^T / sqrt(d)) v̄
    with respect to q̄, k̄, v̄, given d o_CG [m, d]."""
    _, a, _ = compressed_branch(qbar, kbar, vbar)
    return attention_backward(qbar, kbar, vbar, a, do_cg)


def selected_backward(q, k, v, idx, block: int, do_fg):
    """Gradient of the selected branch (one softmax over the union of the
    selected blocks of each query block) given d o_FG [N, d]; the gradients of
    the gathered keys are summed into their tokens."""
    q, k, v, do_fg = _f64(q), _f64(k), _f64(v), _f64(do_fg)
    n_tok, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    within = np.arange(block)
    for i in range(n_tok // block):
        rows = slice(i * block, (i + 1) * block)
        keys = (np.asarray(idx[i], dtype=np.int64)[:, None] * block + within).ravel()
        p = softmax_rows((q[rows] @ k[keys].T) / np.sqrt(d))
        gq, gk, gv = attention_backward(q[rows], k[keys], v[keys], p, do_fg[rows])
        dq[rows] += gq
        np.add.at(dk, keys, gk)
        np.add.at(dv, keys, gv)
    return dq, dk, dv


def local_backward(q, k, v, window: int, do_l, query_chunk: int = 256):
    """Gradient of the local branch given d o_L [N, d]: each query's
    probabilities are those of its own window (reading c12)."""
    q, k, v, do_l = _f64(q), _f64(k), _f64(v), _f64(do_l)
    n_tok, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t0 in range(0, n_tok, query_chunk):
        t1 = min(n_tok, t0 + query_chunk)
        t = np.arange(t0, t1)
        lo, hi = local_window_bounds(t, window, n_tok)
        a, b = int(lo.min()), int(hi.max())
        u = np.arange(a, b)
        s = (q[t0:t1] @ k[a:b].T) / np.sqrt(d)
        inside = (u[None, :] >= lo[:, None]) & (u[None, :] < hi[:, None])
        p = softmax_rows(np.where(inside, s, -np.inf))
        gq, gk, gv = attention_backward(q[t0:t1], k[a:b], v[a:b], p, do_l[t0:t1])
        dq[t0:t1] += gq
        dk[a:b] += gk
        dv[a:b] += gv
    return dq, dk, dv


def bsa_slice_backward(q, k, v, gates, dout, block: int, topn: int, window: int, idx=None) -> dict:
    """Gradient of the BSA forward of one slice (``oracle.bsa.bsa_slice_ref``)
    with respect to q, k, v [N, d] and gates [N, 3], given dout [N, d].

    ``idx`` fixes the selection ([m, n]); by default it is the forward's own
    top-n (reading g1).  Returns dq, dk, dv, dgates and the forward pieces."""
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(gates), _f64(dout)
    n_tok, d = q.shape
    _check_shape(n_tok, block, topn, window)
    m = n_tok // block
    qbar, kbar, vbar = pool_mean(q, block), pool_mean(k, block), pool_mean(v, block)
    s, _, o_cg = compressed_branch(qbar, kbar, vbar)
    if idx is None:
        idx, _ = select_topn(s, topn)
    idx = np.asarray(idx, dtype=np.int64)

    # forward pieces the gate and branch gradients need
    o_fg = fine_selected_branch(q, k, v, idx, block)
    o_l = local_branch(q, k, v, window)
    o_cg_tok = o_cg[np.arange(n_tok) // block]

    # gated sum (reading g3) and the branch outputs' gradients
    dgates = np.stack([np.sum(do * o_cg_tok, axis=1), np.sum(do * o_fg, axis=1), np.sum(do * o_l, axis=1)], axis=1)
    do_cg = (g[:, 0:1] * do).reshape(m, block, d).sum(axis=1)
    do_fg = g[:, 1:2] * do
    do_l = g[:, 2:3] * do

    dq_s, dk_s, dv_s = selected_backward(q, k, v, idx, block, do_fg)
    dq_l, dk_l, dv_l = local_backward(q, k, v, window, do_l)
    dqb, dkb, dvb = compressed_backward(qbar, kbar, vbar, do_cg)
    dq = dq_s + dq_l + pool_backward(dqb, block)
    dk = dk_s + dk_l + pool_backward(dkb, block)
    dv = dv_s + dv_l + pool_backward(dvb, block)
    return dict(dq=dq, dk=dk, dv=dv, dgates=dgates, idx=idx.astype(np.int32),
                o_cg=o_cg, o_fg=o_fg, o_l=o_l, qbar=qbar, kbar=kbar, vbar=vbar,
                do_cg=do_cg, dqbar=dqb, dkbar=dkb, dvbar=dvb)


def bsa_backward_ref(q, k, v, gates, dout, block: int, topn: int, window: int, idx=None) -> dict:
    """``bsa_slice_backward`` over [b, H, N, d] inputs (gates [b, H, N, 3]).
    Returns dq, dk, dv [b, H, N, d] and dgates [b, H, N, 3], float64."""
    q = np.asarray(q)
    b, h, n_tok, d = q.shape
    dq, dk, dv = (np.empty((b, h, n_tok, d)) for _ in range(3))
    dg = np.empty((b, h, n_tok, 3))
    for bi in range(b):
        for hi in range(h):
            r = bsa_slice_backward(q[bi, hi], k[bi, hi], v[bi, hi], gates[bi, hi], dout[bi, hi], block, topn,
                                   window, None if idx is None else idx[bi, hi])
            dq[bi, hi], dk[bi, hi], dv[bi, hi], dg[bi, hi] = r["dq"], r["dk"], r["dv"], r["dgates"]
    return dict(dq=dq, dk=dk, dv=dv, dgates=dg)
