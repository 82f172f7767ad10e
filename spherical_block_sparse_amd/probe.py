"""ctypes binding of libmosaic_probe.so (include/mosaic_probe.h): measured
ceilings of the GPU, reported by bench.py beside the published peaks.
Argument marshalling only; the probes run in the library's kernels."""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_HERE, "libmosaic_probe.so")
EXPORTED = ("mosaic_probe_read", "mosaic_probe_mfma")
_probe = None


def lib() -> ctypes.CDLL:
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build it with `python -m spherical_block_sparse_amd.build`")
        L = ctypes.CDLL(PROBE_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mosaic_probe_read.restype = I
        L.mosaic_probe_read.argtypes = [P, S, P, I, P]
        L.mosaic_probe_mfma.restype = I
        L.mosaic_probe_mfma.argtypes = [P, I, I, P, P]
        _probe = L
    return _probe


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: hipError {rc}")


def probe_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Streaming read of the whole of `buf` (contiguous, 16-byte aligned, size a multiple of 16 bytes)."""
    assert buf.is_cuda and buf.is_contiguous() and sink.dtype == torch.float32 and sink.numel() >= blocks
    nbytes = buf.numel() * buf.element_size()
    assert nbytes % 16 == 0
    _check(lib().mosaic_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                   torch.cuda.current_stream().cuda_stream), "mosaic_probe_read")


def probe_mfma(sink: torch.Tensor, blocks: int, iters: int, clocks: torch.Tensor | None = None) -> float:
    """Back-to-back bf16 MFMAs; returns the FLOPs the launch performs.  clocks (int64 [blocks, 2]),
    if given, receives each workgroup's shader clocks and 100 MHz ticks."""
    assert sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= blocks
    if clocks is not None:
        assert clocks.is_cuda and clocks.dtype == torch.int64 and clocks.numel() >= 2 * blocks
    _check(lib().mosaic_probe_mfma(sink.data_ptr(), blocks, iters, None if clocks is None else clocks.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream), "mosaic_probe_mfma")
    return float(blocks) * 4 * iters * 8 * 16384
