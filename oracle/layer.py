"""Float64 reference of one BSA encoder layer (the attention operator with its
input and output projections).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy float64.

The papernotes.org ICML2026 notes (关键设计) run several BSA layers at native
HEALPix resolution and mix the three BSA branches with per-token gates; they
give neither the projections nor how the gates are made.  Readings taken:

  l1  one linear map of the layer input gives q, k, v (per head, heads
      side by side: feature h*d + j) and 3 gate logits per head (feature
      3*H*d + 3*h + r for branch r); the gates are their logistic sigmoid.
  l2  the layer output is the input plus a linear map of the heads' BSA
      outputs laid side by side (residual form), no normalisation.
  l3  activations between the steps are bf16, as the attention takes bf16
      q, k, v: q, k, v, the merged attention output and the layer output are
      each rounded once to the nearest bf16 (ties to even); the gates stay
      float.
"""

from __future__ import annotations

import numpy as np

from .bsa import _f64, bsa_forward_ref


def round_bf16(a) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to even), as float64.

    bf16 keeps 8 significant bits: a value in [2^e, 2^(e+1)) is rounded to a
    multiple of 2^(e-7).  Written from that definition: scale by the ulp,
    round half to even, scale back (both scalings are exact).  Zero stays
    zero; magnitudes below the normal range are not expected here."""
    a = _f64(a)
    out = np.zeros_like(a)
    nz = a != 0
    e = np.floor(np.log2(np.abs(a[nz])))
    ulp = np.exp2(e - 7)
    r = np.round(a[nz] / ulp) * ulp          # numpy rounds halves to even
    out[nz] = r
    return out


def layer_in_ref(x, w_in, heads: int, head_dim: int):
    """Reading l1: x [b, N, C], w_in [3Hd + 3H, C] -> q, k, v [b, H, N, d]
    (bf16-rounded, l3) and gates [b, H, N, 3] = sigmoid of the logits."""
    x, w_in = _f64(x), _f64(w_in)
    b, n, _ = x.shape
    hd = heads * head_dim
    z = x @ w_in.T                                       # [b, N, 3Hd + 3H]
    split = lambda a: a.reshape(b, n, heads, head_dim).transpose(0, 2, 1, 3)
    q = round_bf16(split(z[..., :hd]))
    k = round_bf16(split(z[..., hd:2 * hd]))
    v = round_bf16(split(z[..., 2 * hd:3 * hd]))
    logits = z[..., 3 * hd:].reshape(b, n, heads, 3).transpose(0, 2, 1, 3)
    gates = 1.0 / (1.0 + np.exp(-logits))
    return q, k, v, gates


def layer_out_ref(attn, w_out, x):
    """Reading l2: y = x + merge_heads(attn) w_outᵀ, attn [b, H, N, d] rounded
    to bf16 first and y rounded to bf16 (l3)."""
    attn, w_out, x = _f64(attn), _f64(w_out), _f64(x)
    b, h, n, d = attn.shape
    a = round_bf16(attn.transpose(0, 2, 1, 3).reshape(b, n, h * d))
    return round_bf16(x + a @ w_out.T)


def layer_ref(x, w_in, w_out, heads: int, head_dim: int, block: int, topn: int, window: int, idx=None) -> dict:
    """One layer: input projection, the BSA forward (``oracle.bsa``), output
    projection.  ``idx`` optionally forces the selection ([b, H, m, n]).
    Returns y [b, N, C] and the intermediate q, k, v, gates, attn, idx."""
    q, k, v, gates = layer_in_ref(x, w_in, heads, head_dim)
    r = bsa_forward_ref(q, k, v, gates, block, topn, window, idx)
    y = layer_out_ref(r["out"], w_out, x)
    return dict(y=y, q=q, k=k, v=v, gates=gates, attn=r["out"], idx=r["idx"], gap=r["gap"])
