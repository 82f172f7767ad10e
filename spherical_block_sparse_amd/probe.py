"""ctypes binding of libmosaic_probe.so (include/mosaic_probe.h): measured
ceilings of the GPU, reported by bench.py beside the published peaks.
Argument marshalling only; the probes run in the library's kernels."""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_HERE, "libmosaic_probe.so")
EXPORTED = ("mosaic_probe_read", "mosaic_probe_mfma", "mosaic_probe_overlap")
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
        L.mosaic_probe_overlap.restype = I
        L.mosaic_probe_overlap.argtypes = [P, I, I, I, P, P, P]
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


OVERLAP_MODES = ("MFMA work, every wave", "vector work, every wave",
                 "MFMA work on waves 0-3, vector work on waves 4-7", "both, interleaved in every wave",
                 "attention chunk, K and V^T operands from LDS", "attention chunk, operands in registers")


def probe_overlap(sink: torch.Tensor, blocks: int, iters: int, mode: int, clocks: torch.Tensor | None = None,
                  simd: torch.Tensor | None = None) -> None:
    """One launch of the MFMA / vector overlap probe (include/mosaic_probe.h)."""
    assert sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= blocks
    if clocks is not None:
        assert clocks.is_cuda and clocks.dtype == torch.int64 and clocks.numel() >= 8 * blocks
    if simd is not None:
        assert clocks is not None and simd.is_cuda and simd.dtype == torch.int32 and simd.numel() >= 8 * blocks
    _check(lib().mosaic_probe_overlap(sink.data_ptr(), blocks, iters, mode,
                                      None if clocks is None else clocks.data_ptr(),
                                      None if simd is None else simd.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream), "mosaic_probe_overlap")


def overlap_report(blocks: int = 1024, iters: int = 1024, reps: int = 5) -> str:
    """Runs the four overlap modes and returns a text table: the mean launch
    time (HIP events), each wave's shader clocks per iteration, and what the
    split mode would take if one wave's MFMAs and the other's vector work ran
    at the same time (the larger of the two halves) or one after the other
    (their sum)."""
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    simd = torch.zeros(blocks * 8, dtype=torch.int32, device="cuda")
    ms, per_wave = [], []
    for mode in range(6):
        probe_overlap(sink, blocks, iters, mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            probe_overlap(sink, blocks, iters, mode)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / reps)
        probe_overlap(sink, blocks, iters, mode, clocks, simd)
        torch.cuda.synchronize()
        c = clocks.view(blocks, 8).double().cpu() / iters
        per_wave.append((float(c[:, :4].median()), float(c[:, 4:].median())))
    sid = (simd.view(blocks, 8).cpu() >> 4) & 3
    paired = float((sid[:, :4] == sid[:, 4:]).all(dim=1).double().mean())
    t0, t1, t2, t3 = ms[:4]
    lines = [f"blocks {blocks} x 8 waves (one workgroup per compute unit at a time), {iters} iterations per wave",
             f"waves w and w+4 on one SIMD in {100 * paired:.1f}% of the workgroups (HW_ID)", "",
             f"{'mode':<58} {'ms':>8} {'clk/iter w0-3':>14} {'clk/iter w4-7':>14}"]
    for mode in range(6):
        lines.append(f"{mode} {OVERLAP_MODES[mode]:<56} {ms[mode]:>8.3f} {per_wave[mode][0]:>14.1f} {per_wave[mode][1]:>14.1f}")
    lines += ["",
              "mode 2 puts half of mode 0's work and half of mode 1's on every SIMD, one wave of each:",
              f"  if they ran at the same time it would take max(t0, t1)/2 = {max(t0, t1) / 2:.3f} ms;",
              f"  one after the other, (t0 + t1)/2 = {(t0 + t1) / 2:.3f} ms; measured {t2:.3f} ms",
              "mode 3 puts all of both on every wave:",
              f"  one after the other, t0 + t1 = {t0 + t1:.3f} ms; measured {t3:.3f} ms "
              f"({100 * (1 - t3 / (t0 + t1)):.1f}% of the sum hidden)",
              "modes 4 and 5, one 64-key attention chunk per iteration, two waves per SIMD (the older",
              "wave of a SIMD finishes first; the SIMD is busy until the later one is done):",
              f"  SIMD clocks per chunk and wave (half the later wave's clocks per iteration): operands from "
              f"LDS {max(per_wave[4]) / 2:.0f}, from registers {max(per_wave[5]) / 2:.0f}"]
    return "\n".join(lines)


if __name__ == "__main__":
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "overlap":
        print(overlap_report(), flush=True)
    else:
        print("usage: python -m spherical_block_sparse_amd.probe overlap", file=sys.stderr)
        sys.exit(2)
