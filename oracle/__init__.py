"""Float64 CPU oracle for the MOSAIC mesh-aligned block-sparse attention (BSA)
forward pass, its gradient, the encoder layer around it, HEALPix coarsening
and the lat-lon -> HEALPix cross-attention interpolation.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library
(``spherical_block_sparse_amd``) and imports nothing from it.

What it follows (the pages the method is taken from):

* papernotes.org ICML2026 notes on "(Sparse) Attention to the Details",
  section 关键设计 (key designs), items "HEALPix 球面镶嵌 + NESTED 索引" and
  "Mesh-aligned Block-Sparse Attention (BSA)": N = 12*Nside^2 pixels, the
  children of NESTED pixel p are 4p..4p+3, tokens are cut into m contiguous
  NESTED blocks, pooled block summaries, three branches (compressed /
  selected / local) and the gated sum of their outputs.
* the arXiv abstract on the mlsanity.com page of the same paper, and the
  "How" section of the paper-curation page: query blocks share one key/value
  selection.

Where the pages leave a step open, the plainest reading is taken; every such
reading is listed in the module docstring of ``oracle.bsa``.

Parity status: every function here is pinned by ``tests/test_oracle.py`` /
``tests/test_oracle_backward.py`` / ``tests/test_oracle_layer.py`` /
``tests/test_oracle_interp.py`` / ``tests/test_healpix.py`` against
finite differences, an independent autograd derivation, closed forms, library routines (torch's
float64 scaled_dot_product_attention), brute force and invariants.  No
function is "parity unpinned".
"""

from .bsa import (  # noqa: F401
    pool_mean,
    compressed_branch,
    select_topn,
    fine_selected_branch,
    local_branch,
    local_window_bounds,
    combine,
    bsa_slice_ref,
    bsa_forward_ref,
    bsa_rows_ref,
    softmax_rows,
)
from .bsa_backward import (  # noqa: F401
    attention_backward,
    pool_backward,
    compressed_backward,
    selected_backward,
    local_backward,
    bsa_slice_backward,
    bsa_backward_ref,
)
from .layer import round_bf16, layer_in_ref, layer_out_ref, layer_ref  # noqa: F401
from .interp import interp_attention, interp_attention_ref  # noqa: F401
from .healpix import npix, nest_children, nest_parent, descendants, coarsen  # noqa: F401
