"""HEALPix NESTED index facts used by the BSA oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: papernotes.org ICML2026 notes on "(Sparse) Attention to the Details",
关键设计 › "HEALPix 球面镶嵌 + NESTED 索引": the sphere is split into 12
equal-area base pixels, each split recursively into four, giving 12*Nside^2
pixels at resolution Nside; in NESTED order the four children of pixel p are
4p, 4p+1, 4p+2, 4p+3, so spatial neighbours are neighbours in memory.

Consequence used by BSA (reading c16 in the oracle docstring): a contiguous
index block of size B = 4^k starting at a multiple of B is exactly the set of
k-fold descendants of one coarse pixel at Nside / 2^k.
"""

from __future__ import annotations


def npix(nside: int) -> int:
    """Number of pixels (= tokens) at resolution ``nside``: 12 * nside^2."""
    if nside < 1:
        raise ValueError("nside must be >= 1")
    return 12 * nside * nside


def nest_children(p: int) -> list[int]:
    """The four NESTED children of pixel ``p`` one level finer: 4p .. 4p+3."""
    return [4 * p, 4 * p + 1, 4 * p + 2, 4 * p + 3]


def nest_parent(p: int) -> int:
    """The NESTED parent of pixel ``p`` one level coarser (inverse of children)."""
    return p // 4


def descendants(p: int, levels: int) -> list[int]:
    """All descendants of pixel ``p`` ``levels`` levels finer, by applying the
    children rule repeatedly (no closed form is used here, so the contiguity of
    the result is something the tests check, not something assumed)."""
    cur = [p]
    for _ in range(levels):
        nxt = []
        for c in cur:
            nxt.extend(nest_children(c))
        cur = nxt
    return sorted(cur)


def coarsen(x, nside: int, levels: int):
    """A field on the NESTED pixels at ``nside`` (x [..., 12*nside^2, C])
    taken to ``nside / 2^levels``: each coarse pixel's value is the mean of
    its ``levels``-fold descendants (children rule applied ``levels`` times).
    Plain loop over coarse pixels, float64."""
    import numpy as np

    x = np.asarray(x, dtype=np.float64)
    if nside % (1 << levels):
        raise ValueError("nside must be divisible by 2^levels")
    coarse = npix(nside >> levels)
    out = np.empty(x.shape[:-2] + (coarse, x.shape[-1]))
    for p in range(coarse):
        out[..., p, :] = x[..., descendants(p, levels), :].mean(axis=-2)
    return out
