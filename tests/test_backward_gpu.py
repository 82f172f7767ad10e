"""GPU parity of mosaic_bsa_backward against the float64 oracle backward
(``oracle.bsa_backward``), through the C ABI.

Both sides take the same bf16 inputs (the oracle on their float64 values),
the same float32 dout and the same selection (the GPU forward's indices,
which the backward holds fixed), so the comparison is element by element.

Tolerance, from the arithmetic of the kernels: every product is bf16 x bf16
with float32 accumulation; q, k, v are exact bf16 inputs, while dout, the
probabilities and dS = P (g dP - D) are rounded to bf16 (relative error
<= 2^-9 each) before they enter a product.  A gradient element is a sum of
such rounded terms, so its error is a few 2^-9 relative to the sum of the
magnitudes of its terms, not to its (possibly cancelling) value.  The check is
relative L2 per tensor <= 1e-2 and max-abs <= 2e-2 times the tensor's largest
magnitude.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from spherical_block_sparse_amd import BSAConfig, _lib, make_inputs
from spherical_block_sparse_amd.synth import to_f64

from parity import log

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2


def _run(cfg: BSAConfig, seed: int = 0):
    dev = "cuda"
    q, k, v, g = make_inputs(cfg, device=dev)
    gen = torch.Generator(device=dev).manual_seed(1000 + cfg.seed + seed)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32)
    _, sel = _lib.mosaic_bsa_forward(q, k, v, g, cfg.nside, cfg.block, cfg.topn, cfg.window)
    dq, dk, dv, dg = _lib.mosaic_bsa_backward(q, k, v, g, sel, dout, cfg.nside, cfg.block, cfg.topn, cfg.window)
    torch.cuda.synchronize()
    ref = oracle.bsa_backward_ref(to_f64(q), to_f64(k), to_f64(v), g.double().cpu().numpy(),
                                  dout.double().cpu().numpy(), cfg.block, cfg.topn, cfg.window,
                                  idx=sel.cpu().numpy())
    out = dict(dq=dq, dk=dk, dv=dv, dgates=dg)
    errs = {}
    for name, t in out.items():
        got = t.double().cpu().numpy()
        want = ref[name]
        assert np.all(np.isfinite(got)), name
        scale = float(np.abs(want).max())
        rel_l2 = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        max_rel = float(np.abs(got - want).max()) / scale
        errs[name] = (rel_l2, max_rel)
        log(f"{cfg.name} {name}: rel-L2 {rel_l2:.3e}, max-abs/max {max_rel:.3e} (max {scale:.3e})")
    for name, (rel_l2, max_rel) in errs.items():
        assert rel_l2 <= REL_L2, (name, rel_l2)
        assert max_rel <= MAX_REL, (name, max_rel)


def test_backward_ns32_two_heads():
    # N = 12288, block 64 (m = 192), top-16, window 256, d = 64
    _run(BSAConfig("ns32-bwd", 32, 1, 2, 64, 64, 16, 256, "iid", 32))


def test_backward_correlated_field_head_dim_32():
    _run(BSAConfig("ns32-d32", 32, 1, 1, 32, 64, 8, 100, "fourier", 33))


def test_backward_block_256():
    # N = 49152, block 256 (m = 192, four 64-query chunks per block), top-4
    _run(BSAConfig("ns64-b256", 64, 1, 1, 64, 256, 4, 300, "fourier", 34))
