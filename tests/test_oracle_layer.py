"""Pins of the float64 encoder-layer oracle (``oracle.layer``) to things other
than itself: torch's float32 -> bfloat16 conversion (a library routine) for
the rounding, hand-made projection weights whose result is known exactly,
and a zero-query layer whose attention reduces to plain means."""

from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import layer_in_ref, layer_out_ref, layer_ref, local_window_bounds, round_bf16


def test_round_bf16_matches_torch_on_float32_inputs():
    # a float32 value rounds to bfloat16 once, so torch's conversion is the exact nearest-even result
    r = np.random.default_rng(0)
    a = (r.standard_normal(200000) * np.exp2(r.integers(-30, 30, 200000))).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(a.astype(np.float64)), want)


def test_round_bf16_ties_go_to_even():
    ulp = 2.0 ** -7   # bf16 spacing in [1, 2)
    np.testing.assert_array_equal(round_bf16([1 + ulp / 2, 1 + 3 * ulp / 2, -(1 + ulp / 2), 0.0, 2.0 + 2 * ulp]),
                                  [1.0, 1 + 2 * ulp, -1.0, 0.0, 2.0 + 2 * ulp])
    # just off a tie rounds to the nearer side (a double rounding through float32 would not)
    assert round_bf16([-2775.999903869452])[0] == -2768.0


def _bf16(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def test_layer_in_identity_weights_copy_channels():
    b, n, h, d = 2, 48, 2, 4
    c = 3 * h * d
    x = _bf16(np.random.default_rng(1).standard_normal((b, n, c)))
    w = np.zeros((3 * h * d + 3 * h, c))
    w[:3 * h * d, :] = np.eye(3 * h * d)                # q, k, v features copy channels 0..3Hd-1
    w[3 * h * d + 1, 5] = 1.0                           # head 0, branch 1 gate logit = x[..., 5]
    q, k, v, g = layer_in_ref(x, w, h, d)
    for t, base in ((q, 0), (k, h * d), (v, 2 * h * d)):
        for hh in range(h):
            np.testing.assert_array_equal(t[:, hh], x[:, :, base + hh * d: base + (hh + 1) * d])
    np.testing.assert_array_equal(g[:, :, :, 0], 0.5)  # zero logits
    np.testing.assert_allclose(g[:, 0, :, 1], expit(x[:, :, 5]), rtol=1e-15)
    np.testing.assert_array_equal(g[:, 1], 0.5)


def test_layer_in_projection_matches_library_matmul():
    b, n, h, d, c = 1, 48, 2, 8, 64
    r = np.random.default_rng(2)
    x, w = r.standard_normal((b, n, c)), r.standard_normal((3 * h * d + 3 * h, c)) / 8
    q, k, v, g = layer_in_ref(x, w, h, d)
    z = (torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
    zk = z[..., h * d:2 * h * d].reshape(b, n, h, d).transpose(0, 2, 1, 3)
    assert np.max(np.abs(k - zk) / np.maximum(np.abs(zk), 1e-30)) <= 2.0 ** -8
    np.testing.assert_allclose(g, expit(z[..., 3 * h * d:].reshape(b, n, h, 3).transpose(0, 2, 1, 3)), rtol=1e-14)


def test_layer_out_zero_weights_and_identity_merge():
    b, n, h, d = 1, 48, 2, 8
    r = np.random.default_rng(3)
    x = _bf16(r.standard_normal((b, n, h * d)))
    attn = r.standard_normal((b, h, n, d))
    np.testing.assert_array_equal(layer_out_ref(attn, np.zeros((h * d, h * d)), x), x)
    # identity output weights and zero input: y is the merged heads, feature h*d + j
    y = layer_out_ref(attn, np.eye(h * d), np.zeros_like(x))
    for hh in range(h):
        np.testing.assert_array_equal(y[:, :, hh * d:(hh + 1) * d], round_bf16(attn[:, hh]))


def test_zero_query_layer_reduces_to_means():
    # q = k = 0: every compressed score ties (selection 0..n-1), every softmax is uniform,
    # so the branches are the global mean of v, the mean of blocks 0..n-1 and the window mean
    nside, b, h, d, block, topn, window = 2, 1, 2, 4, 4, 3, 5
    n = 12 * nside * nside
    c = 16
    r = np.random.default_rng(4)
    x = _bf16(r.standard_normal((b, n, c)))
    w_in = np.zeros((3 * h * d + 3 * h, c))
    w_in[2 * h * d:3 * h * d] = _bf16(r.standard_normal((h * d, c)) / 4)     # only v and the gates
    w_in[3 * h * d:] = _bf16(r.standard_normal((3 * h, c)) / 4)
    w_out = _bf16(r.standard_normal((c, h * d)) / 4)
    got = layer_ref(x, w_in, w_out, h, d, block, topn, window)
    np.testing.assert_array_equal(got["idx"], np.tile(np.arange(topn, dtype=np.int32), (b, h, n // block, 1)))

    v = round_bf16((x @ w_in[2 * h * d:3 * h * d].T).reshape(b, n, h, d).transpose(0, 2, 1, 3))
    g = expit((x @ w_in[3 * h * d:].T).reshape(b, n, h, 3).transpose(0, 2, 1, 3))
    o_cg = v.mean(axis=2, keepdims=True)
    o_fg = v[:, :, :topn * block].mean(axis=2, keepdims=True)
    lo, hi = local_window_bounds(np.arange(n), window, n)
    cs = np.concatenate([np.zeros((b, h, 1, d)), np.cumsum(v, axis=2)], axis=2)
    o_l = (cs[:, :, hi] - cs[:, :, lo]) / (hi - lo)[None, None, :, None]
    attn = g[..., 0:1] * o_cg + g[..., 1:2] * o_fg + g[..., 2:3] * o_l
    np.testing.assert_allclose(got["attn"], attn, rtol=1e-12, atol=1e-14)
    merged = round_bf16(attn.transpose(0, 2, 1, 3).reshape(b, n, h * d))
    y = round_bf16(x + merged @ w_out.T)
    # ties of the final rounding aside, y agrees exactly
    assert np.mean(got["y"] == y) > 0.999
    np.testing.assert_allclose(got["y"], y, rtol=2.0 ** -7, atol=0)
