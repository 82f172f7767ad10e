"""Selection locality of BSA under NESTED vs latitude-longitude (RING) token order.

    python -m spherical_block_sparse_amd.locality_study [--config ns128] [--steps 10]

The notes page (papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED and
› BSA) credits NESTED order with making every block one compact coarse pixel
and its reads coalesced, and its ablation replaces HEALPix blocks with
latitude-longitude blocks.  This runs the same BSA forward on the same
synthetic field twice: tokens in NESTED order, and the same tokens in RING
order (iso-latitude rings, the layout of a lat-lon raster), where a block of
B consecutive tokens is a strip along a ring and the window follows the ring.

Printed as one JSON line per order:
  * block_radius_deg: mean over blocks of the largest angle between a
    token's pixel centre and its block's mean direction (compactness);
  * select_jaccard: mean Jaccard index of the selected key-block sets of
    consecutive query blocks (how much K/V the next tile re-reads);
  * select_footprint: distinct key blocks selected by each run of 128
    consecutive query blocks, over 128*n (the L2 working set of the
    query tiles one XCD runs together; lower = more reuse);
  * fine_ms / forward_ms: the fine kernel and the whole forward, HIP events.
HBM traffic of the two orders comes from rocprofv3 FETCH_SIZE passes over
``profile_run --order nested|ring``.
"""

from __future__ import annotations

import argparse
import json
import sys

import numpy as np
import torch

from . import CONFIGS, make_inputs
from . import _lib
from .synth import nest_ring_order, pix2vec_nest


def permute_tokens(tensors, perm):
    """The same tensors with the token axis (dim 2) reordered: position i
    holds NESTED pixel perm[i]."""
    idx = torch.as_tensor(perm, device=tensors[0].device, dtype=torch.long)
    return [t.index_select(2, idx).contiguous() for t in tensors]


def block_radius_deg(vec: np.ndarray, block: int) -> float:
    m = vec.shape[0] // block
    v = vec.reshape(m, block, 3)
    c = v.mean(axis=1)
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    cosang = np.clip(np.einsum("mbk,mk->mb", v, c), -1.0, 1.0)
    return float(np.degrees(np.arccos(cosang.min(axis=1))).mean())


def selection_stats(sel: np.ndarray, run: int = 128) -> tuple[float, float]:
    """sel [S, m, n] -> (mean Jaccard of consecutive rows, mean footprint per run of rows)."""
    s, m, n = sel.shape
    jac, foot = [], []
    for si in range(s):
        rows = [set(r.tolist()) for r in sel[si]]
        jac.extend(len(a & b) / len(a | b) for a, b in zip(rows[:-1], rows[1:]))
        for r0 in range(0, m - run + 1, run):
            foot.append(len(set().union(*rows[r0:r0 + run])) / (run * n))
    return float(np.mean(jac)), float(np.mean(foot))


def time_ms(fn, steps: int) -> float:
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="ns128", choices=sorted(CONFIGS))
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--stat-slices", type=int, default=8, help="slices the CPU statistics use")
    args = ap.parse_args()
    cfg = CONFIGS[args.config]
    q, k, v, g = make_inputs(cfg, device="cuda")
    vec = pix2vec_nest(cfg.nside)
    perm = nest_ring_order(cfg.nside)
    for order in ("nested", "ring"):
        if order == "ring":
            q, k, v, g = permute_tokens([q, k, v, g], perm)
            vec = vec[perm]
        out, sel = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
        knorm = torch.empty((cfg.batch, cfg.heads, cfg.n_blocks), dtype=torch.float32, device=q.device)
        qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm)
        o_cg, sel2 = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn)
        sb = _lib.mosaic_bsa_select_bound(sel2, knorm, cfg.nside, cfg.block, cfg.topn, cfg.head_dim)
        fine = lambda: _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel2, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                            out, knorm=knorm, sel_bound=sb)
        fwd = lambda: _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window, out, sel)
        fine_ms, fwd_ms = time_ms(fine, args.steps), time_ms(fwd, args.steps)
        s = sel.view(-1, cfg.n_blocks, cfg.topn)[: args.stat_slices].cpu().numpy()
        jac, foot = selection_stats(s)
        print(json.dumps({"config": cfg.name, "order": order, "block": cfg.block,
                          "block_radius_deg": block_radius_deg(vec, cfg.block),
                          "select_jaccard": jac, "select_footprint": foot,
                          "fine_ms": fine_ms, "forward_ms": fwd_ms, "stat_slices": int(s.shape[0])}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
