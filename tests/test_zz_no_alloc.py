"""mosaic_bsa_forward_noalloc (the forward with the library's static device
scratch as its workspace) against mosaic_bsa_forward, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (the scratch
keeps the first call's contents), each compared bit for bit with the
workspace entry point on the same inputs: the same kernels run on the same
data, so indices and outputs must be identical.  A shape whose workspace
exceeds the scratch is rejected before anything is launched.
"""

from __future__ import annotations

import pytest
import torch

from spherical_block_sparse_amd import CONFIGS, _lib, make_inputs
from spherical_block_sparse_amd._lib import MosaicError

from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_noalloc_equals_forward_on_two_calls_second_smaller():
    big = CONFIGS["ns64"]                      # 38 MB of workspace
    small = CONFIGS["ns32"].with_(heads=3)     # smaller: m = 192, 3 slices
    cases = []
    for cfg in (big, small):
        log(f"[case] {cfg.name}: b={cfg.batch} H={cfg.heads} nside={cfg.nside} block={cfg.block} topn={cfg.topn}")
        q, k, v, g = make_inputs(cfg, device=DEV)
        out_ref, idx_ref = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
        cases.append((cfg, (q, k, v, g), out_ref, idx_ref))
    torch.cuda.synchronize()
    results = []
    for cfg, (q, k, v, g), _, _ in cases:   # the two allocation-free calls back to back
        results.append(_lib.mosaic_bsa_forward_noalloc(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window))
    torch.cuda.synchronize()
    for (cfg, _, out_ref, idx_ref), (out, idx) in zip(cases, results):
        assert torch.equal(idx, idx_ref), cfg.name
        assert torch.equal(out, out_ref), cfg.name
        log(f"    {cfg.name}: indices and outputs identical to mosaic_bsa_forward")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    cfg = CONFIGS["ns128"]
    q = torch.empty((cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((cfg.batch, cfg.heads, cfg.n_tokens, 3), dtype=torch.float32, device=DEV)
    with pytest.raises(MosaicError, match="static scratch"):
        _lib.mosaic_bsa_forward_noalloc(q, q, q, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
