"""Run one BSA stage (or a plain copy) a few times, for rocprofv3 passes.

    python -m spherical_block_sparse_amd.profile_run --config ns128 --stage fine --reps 2
    python -m spherical_block_sparse_amd.profile_run --copy-mib 4096 --reps 2

--stage pool | select | fine | forward | train | layer_in | layer runs that
entry point (the layer stages with 512 channels)
`reps` times on the workload's synthetic inputs (the earlier stages run once
beforehand to produce their inputs); --stage backward runs the training
forward once and then the backward from its saved state `reps` times, with
a seeded float32 upstream gradient.  --order ring lays the same field out in
RING (iso-latitude) token order.  --copy-mib N copies an N MiB buffer
`reps` times (torch's copy_ of a contiguous tensor: the runtime's device copy
kernel): N MiB read and N MiB written per call, the calibration of the
FETCH_SIZE / WRITE_SIZE counters.
"""

from __future__ import annotations

import argparse
import sys

import torch

from . import CONFIGS, make_inputs
from . import _lib


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="ns128", choices=sorted(CONFIGS))
    ap.add_argument("--stage", default="fine",
                    choices=["pool", "select", "fine", "forward", "train", "backward", "layer_in", "layer"])
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--order", default="nested", choices=["nested", "ring"],
                    help="token order of the inputs (ring: the same field laid out by iso-latitude rings)")
    args = ap.parse_args()

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.copy_mib} MiB x {args.reps}", flush=True)
        return 0

    cfg = CONFIGS[args.config]
    if args.stage in ("layer_in", "layer"):   # the encoder layer of 512 channels on the workload's mesh
        from . import make_layer_inputs
        x, w_in, w_out = make_layer_inputs(cfg, 512, device="cuda")
        for _ in range(args.reps):
            if args.stage == "layer_in":
                _lib.mosaic_bsa_layer_in(x, w_in[0], cfg.heads, cfg.head_dim, cfg.nside)
            else:
                _lib.mosaic_bsa_layer_forward(x, w_in[0], w_out[0], cfg.heads, cfg.head_dim, cfg.nside, cfg.block,
                                              cfg.topn, cfg.window)
        torch.cuda.synchronize()
        print(f"{args.stage} {cfg.name} x {args.reps} done", flush=True)
        return 0
    q, k, v, g = make_inputs(cfg, device="cuda", dtype=torch.bfloat16)
    if args.order == "ring":
        from .locality_study import permute_tokens
        from .synth import nest_ring_order
        q, k, v, g = permute_tokens([q, k, v, g], nest_ring_order(cfg.nside))
    b, h, m, d = cfg.batch, cfg.heads, cfg.n_blocks, cfg.head_dim
    knorm = torch.empty((b, h, m), dtype=torch.float32, device="cuda")
    kp = torch.empty((b, h, m, 2, d), dtype=torch.bfloat16, device="cuda")   # the forward's extra pool outputs
    kb2 = torch.empty((b, h, m), dtype=torch.float32, device="cuda")
    qbar, kbar, vbar = _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, knorm=knorm, kpieces=kp, kbn2=kb2)
    o_cg, sel = _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn, kpieces=kp,
                                                kbn2=kb2)
    sb = _lib.mosaic_bsa_select_bound(sel, knorm, cfg.nside, cfg.block, cfg.topn, d)
    torch.cuda.synchronize()
    if args.stage == "backward":
        _, sel_t, saved = _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
        gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 7)
        dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32)
        grads = _lib.mosaic_bsa_backward(q, k, v, g, sel_t, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                         saved=saved)
        torch.cuda.synchronize()
    for _ in range(args.reps):
        if args.stage == "backward":
            _lib.mosaic_bsa_backward(q, k, v, g, sel_t, dout, cfg.nside, cfg.block, cfg.topn, cfg.window,
                                     *grads, saved=saved)
        elif args.stage == "train":
            _lib.mosaic_bsa_forward_train(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
        elif args.stage == "pool":
            _lib.mosaic_bsa_pool(q, k, v, cfg.nside, cfg.block, qbar, kbar, vbar, knorm=knorm, kpieces=kp, kbn2=kb2)
        elif args.stage == "select":
            _lib.mosaic_bsa_compress_select(qbar, kbar, vbar, cfg.nside, cfg.block, cfg.topn, o_cg, sel, kpieces=kp,
                                            kbn2=kb2)
        elif args.stage == "fine":
            _lib.mosaic_bsa_fine(q, k, v, g, o_cg, sel, cfg.nside, cfg.block, cfg.topn, cfg.window, knorm=knorm,
                                 sel_bound=sb)
        else:
            _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    print(f"{args.stage} {cfg.name} x {args.reps} done", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
