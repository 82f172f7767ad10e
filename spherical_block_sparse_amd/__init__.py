"""MI355X (gfx950) implementation of the MOSAIC mesh-aligned block-sparse
attention (BSA) forward pass over HEALPix NESTED tokens.

The compute lives in the C-ABI library ``libmosaic_bsa.so`` (hand-written HIP
kernels, declared in ``include/mosaic_bsa.h``); ``_lib`` is the thin ctypes
binding over it and ``synth`` makes the seeded synthetic inputs.
"""

from .synth import BSAConfig, CONFIGS, make_inputs, make_layer_inputs  # noqa: F401

__all__ = ["BSAConfig", "CONFIGS", "make_inputs", "make_layer_inputs"]
