"""Pins of the float64 oracle backward (``oracle.bsa_backward``) to things
other than itself:

* central finite differences of the oracle forward (``oracle.bsa``) with the
  selection held fixed (reading g1), on every input element of a tiny slice;
* autograd of an independently written dense-mask torch float64 forward
  (pooling by reshape-mean, block and band masks over the full N x N score
  matrix), which shares no code with either oracle module;
* special cases with closed forms: window 1, one-hot gates, top-n = all.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import (
    attention_backward,
    bsa_slice_backward,
    bsa_slice_ref,
    local_backward,
    selected_backward,
    softmax_rows,
)


def _inputs(n_tok, d, seed):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((n_tok, d)) for _ in range(3))
    g = 1.0 / (1.0 + np.exp(-r.standard_normal((n_tok, 3))))
    do = r.standard_normal((n_tok, d))
    return q, k, v, g, do


def test_attention_backward_matches_finite_differences():
    r = np.random.default_rng(3)
    q, k, v, do = r.standard_normal((5, 4)), r.standard_normal((7, 4)), r.standard_normal((7, 3)), r.standard_normal((5, 3))
    mask = r.random((5, 7)) < 0.7
    mask[:, 0] = True

    def loss(q, k, v):
        s = np.where(mask, q @ k.T / 2.0, -np.inf)
        return float(np.sum((softmax_rows(s) @ v) * do))

    p = softmax_rows(np.where(mask, q @ k.T / 2.0, -np.inf))
    dq, dk, dv = attention_backward(q, k, v, p, do)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for ix in np.ndindex(*x.shape):
            x0 = x[ix]
            x[ix] = x0 + eps
            lp = loss(q, k, v)
            x[ix] = x0 - eps
            lm = loss(q, k, v)
            x[ix] = x0
            num[ix] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_bsa_backward_finite_differences_every_element():
    # nside 2: N = 48, d = 4, 12 blocks of 4, top-3, window 5
    n_tok, d, block, topn, window = 48, 4, 4, 3, 5
    q, k, v, g, do = _inputs(n_tok, d, 11)
    idx = bsa_slice_ref(q, k, v, g, block, topn, window)["idx"]
    ref = bsa_slice_backward(q, k, v, g, do, block, topn, window)
    np.testing.assert_array_equal(ref["idx"], idx)

    def loss():
        return float(np.sum(bsa_slice_ref(q, k, v, g, block, topn, window, idx=idx)["out"] * do))

    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dgates", g)):
        num = np.zeros_like(x)
        for ix in np.ndindex(*x.shape):
            x0 = x[ix]
            x[ix] = x0 + eps
            lp = loss()
            x[ix] = x0 - eps
            lm = loss()
            x[ix] = x0
            num[ix] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(ref[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_forward(q, k, v, g, block, window, idx):
    """Dense-mask float64 forward: every branch as a masked softmax over the
    full N x N matrix.  Written independently of ``oracle.bsa``."""
    n_tok, d = q.shape
    m = n_tok // block
    blk = torch.arange(n_tok) // block
    qb, kb, vb = (x.reshape(m, block, d).mean(dim=1) for x in (q, k, v))
    o_cg = torch.softmax(qb @ kb.T / math.sqrt(d), dim=-1) @ vb
    s = q @ k.T / math.sqrt(d)
    chosen = torch.zeros(m, m, dtype=torch.bool)
    chosen[torch.arange(m)[:, None], torch.as_tensor(idx, dtype=torch.long)] = True
    sel_mask = chosen[blk][:, blk]
    t = torch.arange(n_tok)
    band = (t[None, :] >= t[:, None] - window // 2) & (t[None, :] < t[:, None] + (window + 1) // 2)
    o_fg = torch.softmax(s.masked_fill(~sel_mask, -math.inf), dim=-1) @ v
    o_l = torch.softmax(s.masked_fill(~band, -math.inf), dim=-1) @ v
    return g[:, 0:1] * o_cg[blk] + g[:, 1:2] * o_fg + g[:, 2:3] * o_l


@pytest.mark.parametrize("n_tok,d,block,topn,window", [(192, 8, 16, 3, 9), (192, 8, 4, 5, 20), (48, 4, 16, 3, 200)])
def test_bsa_backward_matches_autograd_of_dense_forward(n_tok, d, block, topn, window):
    q, k, v, g, do = _inputs(n_tok, d, 5 + block)
    ref = bsa_slice_backward(q, k, v, g, do, block, topn, window)
    tq, tk, tv, tg = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g))
    out = _torch_forward(tq, tk, tv, tg, block, window, ref["idx"])
    np.testing.assert_allclose(out.detach().numpy(), bsa_slice_ref(q, k, v, g, block, topn, window)["out"],
                               rtol=1e-12, atol=1e-12)
    grads = torch.autograd.grad((out * torch.tensor(do)).sum(), (tq, tk, tv, tg))
    for name, gr in zip(("dq", "dk", "dv", "dgates"), grads):
        np.testing.assert_allclose(ref[name], gr.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_window_one_local_gradient_is_gated_identity():
    # a one-key window gives o_L = v: dv = g_L dO, no q or k gradient
    q, k, v, g, do = _inputs(48, 4, 2)
    dq, dk, dv = local_backward(q, k, v, 1, g[:, 2:3] * do)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, g[:, 2:3] * do, rtol=0, atol=1e-15)


def test_one_hot_gates_isolate_branches():
    n_tok, d, block, topn, window = 192, 8, 16, 3, 9
    q, k, v, _, do = _inputs(n_tok, d, 4)
    for branch in range(3):
        g = np.zeros((n_tok, 3))
        g[:, branch] = 1.0
        r = bsa_slice_backward(q, k, v, g, do, block, topn, window)
        if branch == 0:   # compressed only: every token of a block gets the same dq, dk, dv
            for x in ("dq", "dk", "dv"):
                blocks = r[x].reshape(n_tok // block, block, d)
                np.testing.assert_allclose(blocks, blocks[:, :1, :].repeat(block, axis=1), rtol=0, atol=1e-15)
        if branch == 1:   # selected only: equals selected_backward with dO
            dq, dk, dv = selected_backward(q, k, v, r["idx"], block, do)
            np.testing.assert_allclose(r["dq"], dq, atol=1e-13)
            np.testing.assert_allclose(r["dk"], dk, atol=1e-13)
            np.testing.assert_allclose(r["dv"], dv, atol=1e-13)
        if branch == 2:   # local only
            dq, dk, dv = local_backward(q, k, v, window, do)
            np.testing.assert_allclose(r["dq"], dq, atol=1e-13)
            np.testing.assert_allclose(r["dv"], dv, atol=1e-13)


def test_selected_all_blocks_is_dense_attention_gradient():
    n_tok, d, block = 48, 4, 4
    q, k, v, _, do = _inputs(n_tok, d, 9)
    m = n_tok // block
    idx = np.tile(np.arange(m), (m, 1))
    dq, dk, dv = selected_backward(q, k, v, idx, block, do)
    p = softmax_rows(q @ k.T / math.sqrt(d))
    eq, ek, ev = attention_backward(q, k, v, p, do)
    np.testing.assert_allclose(dq, eq, atol=1e-13)
    np.testing.assert_allclose(dk, ek, atol=1e-13)
    np.testing.assert_allclose(dv, ev, atol=1e-13)


def test_gate_gradients_sum_rule():
    # sum_t dg_t . g_t == sum_t dO_t . out_t (the output is linear in the gates)
    n_tok, d, block, topn, window = 192, 8, 16, 3, 9
    q, k, v, g, do = _inputs(n_tok, d, 12)
    r = bsa_slice_backward(q, k, v, g, do, block, topn, window)
    out = bsa_slice_ref(q, k, v, g, block, topn, window)["out"]
    assert abs(np.sum(r["dgates"] * g) - np.sum(do * out)) < 1e-10
