"""Float64 reference of the BSA forward pass, one (batch, head) slice at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy float64;
no blocking, fusion or reordering beyond what the definition states.

Definition followed: papernotes.org ICML2026 notes on "(Sparse) Attention to
the Details", 关键设计 › "Mesh-aligned Block-Sparse Attention (BSA)" (核心思路):
the N tokens, in HEALPix NESTED order, are cut into m non-overlapping blocks;
a pooling phi gives block summaries q̄_i, k̄_j, v̄_j; three branches are mixed
by gates g_CG, g_FG, g_L:

  (a) compressed: ā_ij = softmax_j(q̄_i·k̄_j / sqrt(d_k)), block-to-block
      attention whose result is broadcast to every token of query block i;
  (b) selected: each query block takes the top-n key blocks by the
      compressed scores and runs full-resolution attention over the tokens of
      those blocks (the selection is shared by the block -- also stated in
      the mlsanity.com abstract and the paper-curation page's "How" section);
  (c) local: standard attention of each query over a sliding window;
  out_t = g_CG·o_CG + g_FG·o_FG + g_L·o_L.

Readings taken where the pages are silent or ambiguous:

  c1  pooling phi = arithmetic mean over the block's tokens, no weights.
  c2  the compressed branch uses block-level q̄_i; its output for block i,
      o_CG_i = sum_j ā_ij v̄_j, is the same for every token of block i.
  c3  no causal mask anywhere (spherical data has no direction).
  c4  scale 1/sqrt(d) with d = head_dim, in every branch.
  c5  selection ranks the logits s_ij = q̄_i·k̄_j/sqrt(d) (same order as ā_ij,
      without the round-off of the probabilities).
  c6  ties in s_ij go to the lower block index.
  c7  no forced blocks (own block, neighbours): pure top-n.
  c8  selected indices are returned in ascending block order.
  c11 the selected branch is ONE softmax over the union of the n·B selected
      tokens (no per-block normalisation).
  c12 local window of query t = [t - floor(W/2), t + ceil(W/2)), i.e. W keys
      centred on t including t, clipped to [0, N) with no wraparound.
  c13 branches are independent: a key may appear in both the selected blocks
      and the window and counts in both softmaxes.
  c14 gates are inputs, not normalised across branches.
  c15 every (batch, head) slice has its own pooling, scores and selection.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis.  Entries equal to -inf are excluded keys
    (probability 0).  Every row must hold at least one finite entry."""
    x = _f64(x)
    mx = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - mx)
    return e / np.sum(e, axis=-1, keepdims=True)


def pool_mean(x: np.ndarray, block: int) -> np.ndarray:
    """Pooling phi (reading c1): mean of each block of ``block`` consecutive
    NESTED tokens.  x: [N, d] -> [m, d], m = N / block."""
    x = _f64(x)
    n, d = x.shape
    if n % block:
        raise ValueError("N must be a multiple of the block size")
    return x.reshape(n // block, block, d).mean(axis=1)


def compressed_branch(qbar: np.ndarray, kbar: np.ndarray, vbar: np.ndarray):
    """Compressed branch (a): logits s = q̄ k̄^T / sqrt(d), ā = row softmax of s,
    o_CG = ā v̄ (one row per query block).  Returns (s, ā, o_CG)."""
    qbar, kbar, vbar = _f64(qbar), _f64(kbar), _f64(vbar)
    d = qbar.shape[1]
    s = (qbar @ kbar.T) / np.sqrt(d)
    a = softmax_rows(s)
    return s, a, a @ vbar


def select_topn(s: np.ndarray, topn: int):
    """Top-n key blocks per query block from the compressed logits (b, c5-c8).

    Order each row by descending logit; a stable sort keeps equal logits in
    ascending block order, so ties go to the lower index (c6).  The first n
    are returned in ascending block order (c8).

    Returns (idx [rows, n] int32, gap [rows] float64) where gap is the logit
    difference between the n-th and (n+1)-th entries of the sorted row
    (+inf when n equals the number of blocks).  gap decides which rows count
    as near-ties when comparing against another implementation.
    """
    s = _f64(s)
    rows, m = s.shape
    if not 1 <= topn <= m:
        raise ValueError("topn must lie in [1, m]")
    order = np.argsort(-s, axis=1, kind="stable")
    idx = np.sort(order[:, :topn], axis=1).astype(np.int32)
    if topn == m:
        gap = np.full(rows, np.inf)
    else:
        r = np.arange(rows)
        gap = s[r, order[:, topn - 1]] - s[r, order[:, topn]]
    return idx, gap


def fine_selected_branch(q, k, v, idx, block: int) -> np.ndarray:
    """Selected branch (b, c11): every token t of query block i attends, with
    one softmax, to all tokens of the key blocks idx[i]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_tok, d = q.shape
    m = n_tok // block
    out = np.empty((n_tok, v.shape[1]))
    within = np.arange(block)
    for i in range(m):
        keys = (np.asarray(idx[i], dtype=np.int64)[:, None] * block + within).ravel()
        s = (q[i * block:(i + 1) * block] @ k[keys].T) / np.sqrt(d)
        out[i * block:(i + 1) * block] = softmax_rows(s) @ v[keys]
    return out


def local_window_bounds(t, window: int, n_tok: int):
    """Window of query t (reading c12): [t - floor(W/2), t + ceil(W/2)) ∩ [0, N)."""
    t = np.asarray(t)
    lo = np.maximum(t - window // 2, 0)
    hi = np.minimum(t + (window + 1) // 2, n_tok)
    return lo, hi


def local_branch(q, k, v, window: int, query_chunk: int = 256) -> np.ndarray:
    """Local branch (c, c12): each query attends to the keys of its own window.

    Queries are handled a batch at a time for speed; inside a batch each row's
    keys are exactly its own window (the others are set to -inf)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_tok, d = q.shape
    if window < 1:
        raise ValueError("window must be >= 1")
    out = np.empty((n_tok, v.shape[1]))
    for t0 in range(0, n_tok, query_chunk):
        t1 = min(n_tok, t0 + query_chunk)
        t = np.arange(t0, t1)
        lo, hi = local_window_bounds(t, window, n_tok)
        a, b = int(lo.min()), int(hi.max())
        u = np.arange(a, b)
        s = (q[t0:t1] @ k[a:b].T) / np.sqrt(d)
        inside = (u[None, :] >= lo[:, None]) & (u[None, :] < hi[:, None])
        s = np.where(inside, s, -np.inf)
        out[t0:t1] = softmax_rows(s) @ v[a:b]
    return out


def combine(gates, o_cg_blocks, o_fg, o_l, block: int) -> np.ndarray:
    """Gated sum (c14): out_t = g_t0·o_CG[t // B] + g_t1·o_FG_t + g_t2·o_L_t."""
    g = _f64(gates)
    n_tok = g.shape[0]
    o_cg_tok = _f64(o_cg_blocks)[np.arange(n_tok) // block]
    return g[:, 0:1] * o_cg_tok + g[:, 1:2] * _f64(o_fg) + g[:, 2:3] * _f64(o_l)


def _check_shape(n_tok: int, block: int, topn: int, window: int):
    if n_tok % 12:
        raise ValueError("N must be 12*Nside^2")
    nside = int(round((n_tok // 12) ** 0.5))
    if 12 * nside * nside != n_tok:
        raise ValueError("N must be 12*Nside^2")
    if block < 1 or n_tok % block:
        raise ValueError("block must divide N")
    m = n_tok // block
    if not 1 <= topn <= m:
        raise ValueError("topn must lie in [1, m]")
    if window < 1:
        raise ValueError("window must be >= 1")


def bsa_slice_ref(q, k, v, gates, block: int, topn: int, window: int, idx=None) -> dict:
    """BSA forward for one (batch, head) slice.

    q, k, v: [N, d]; gates: [N, 3] = (g_CG, g_FG, g_L).  When ``idx`` is given
    ([m, n] block indices) the selected branch uses it instead of its own
    top-n ("forced" mode, used to compare outputs on near-tie rows).

    Returns a dict with out [N, d], idx [m, n] int32, gap [m], s [m, m],
    qbar/kbar/vbar [m, d], o_cg [m, d] (per block), o_fg [N, d], o_l [N, d].
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gates)
    n_tok = q.shape[0]
    _check_shape(n_tok, block, topn, window)
    qbar, kbar, vbar = pool_mean(q, block), pool_mean(k, block), pool_mean(v, block)
    s, _, o_cg = compressed_branch(qbar, kbar, vbar)
    own_idx, gap = select_topn(s, topn)
    use_idx = own_idx if idx is None else np.asarray(idx, dtype=np.int64)
    o_fg = fine_selected_branch(q, k, v, use_idx, block)
    o_l = local_branch(q, k, v, window)
    out = combine(g, o_cg, o_fg, o_l, block)
    return dict(out=out, idx=own_idx, gap=gap, s=s, qbar=qbar, kbar=kbar, vbar=vbar,
                o_cg=o_cg, o_fg=o_fg, o_l=o_l)


def bsa_forward_ref(q, k, v, gates, block: int, topn: int, window: int, idx=None) -> dict:
    """BSA forward for [b, H, N, d] inputs (gates [b, H, N, 3]), slice by slice.

    Returns out [b, H, N, d] float64, idx [b, H, m, n] int32, gap [b, H, m]."""
    q = np.asarray(q)
    b, h, n_tok, d = q.shape
    m = n_tok // block
    out = np.empty((b, h, n_tok, v.shape[-1]))
    idx_out = np.empty((b, h, m, topn), np.int32)
    gap = np.empty((b, h, m))
    for bi in range(b):
        for hi in range(h):
            r = bsa_slice_ref(q[bi, hi], k[bi, hi], v[bi, hi], gates[bi, hi], block, topn, window,
                              None if idx is None else idx[bi, hi])
            out[bi, hi], idx_out[bi, hi], gap[bi, hi] = r["out"], r["idx"], r["gap"]
    return dict(out=out, idx=idx_out, gap=gap)


def bsa_rows_ref(q, k, v, gates, block: int, topn: int, window: int, tokens, idx=None) -> dict:
    """BSA forward of one slice evaluated at the listed query tokens only.

    Same definition as ``bsa_slice_ref`` (pooling over every block, the full
    row of compressed logits of each needed query block, the top-n of that
    row, the selected blocks and the window of each listed token), for
    checking large inputs on a sample of outputs.  ``idx`` optionally forces
    the selection ([m, n], only the rows of the needed query blocks are read).

    Returns out [T, d], and for every distinct query block touched: its idx
    row and gap, keyed by block index.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(gates)
    n_tok, d = q.shape
    _check_shape(n_tok, block, topn, window)
    tokens = np.asarray(tokens, dtype=np.int64)
    kbar, vbar = pool_mean(k, block), pool_mean(v, block)
    blocks = np.unique(tokens // block)
    qbar_rows = q.reshape(n_tok // block, block, d)[blocks].mean(axis=1)
    s, _, o_cg = compressed_branch(qbar_rows, kbar, vbar)
    own_idx, gap = select_topn(s, topn)
    row_of = {int(bk): r for r, bk in enumerate(blocks)}
    out = np.empty((tokens.size, v.shape[1]))
    within = np.arange(block)
    for ti, t in enumerate(tokens):
        r = row_of[int(t // block)]
        sel = own_idx[r] if idx is None else np.asarray(idx[int(t // block)], dtype=np.int64)
        keys = (np.asarray(sel, dtype=np.int64)[:, None] * block + within).ravel()
        p_fg = softmax_rows((k[keys] @ q[t]) / np.sqrt(d))
        lo, hi = local_window_bounds(t, window, n_tok)
        p_l = softmax_rows((k[lo:hi] @ q[t]) / np.sqrt(d))
        out[ti] = g[t, 0] * o_cg[r] + g[t, 1] * (p_fg @ v[keys]) + g[t, 2] * (p_l @ v[lo:hi])
    return dict(out=out,
                idx={int(bk): own_idx[r] for bk, r in row_of.items()},
                gap={int(bk): float(gap[r]) for bk, r in row_of.items()},
                o_cg={int(bk): o_cg[r] for bk, r in row_of.items()})
