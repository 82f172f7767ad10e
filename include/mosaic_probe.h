/* Measurement probes of libmosaic_probe.so: ceilings of the GPU that the
 * BSA kernels' roofline fractions are read against, beside the published
 * peaks.  Not part of the attention method (see mosaic_bsa.h for that).
 *
 * Conventions: device pointers owned by the caller; every call only enqueues
 * work on `stream` (a hipStream_t, NULL = the legacy default stream) and
 * returns a hipError_t value (0 = hipSuccess; hipErrorInvalidValue for a
 * NULL pointer, a misaligned buffer or a non-positive count, checked before
 * any launch).  The result of a probe is its duration, which the caller
 * times with events on the same stream. */
#ifndef MOSAIC_PROBE_H
#define MOSAIC_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16) at `buf` (16-byte aligned) by
 * `blocks` workgroups of 256 threads: 16-byte nontemporal loads, eight in
 * flight per lane, consecutive workgroups on consecutive 4 KB spans.  `sink`
 * (float32 [blocks]) is written only in a case that does not occur; it
 * keeps the loads from being dropped. */
int mosaic_probe_read(const void* buf, size_t bytes, float* sink, int blocks, void* stream);

/* `blocks` workgroups of four waves, each wave issuing `iters` x 8
 * independent v_mfma_f32_16x16x32_bf16 on register operands: 16384 FLOPs
 * per instruction, blocks * 4 * iters * 8 instructions in all.  `sink`
 * (float32 [blocks]) as above.  `clocks` (may be NULL): uint64
 * [blocks][2], each workgroup's elapsed shader clocks (s_memtime) and
 * 100 MHz ticks (s_memrealtime) over its run; their ratio x 100 MHz is the
 * shader clock it ran at. */
int mosaic_probe_mfma(float* sink, int blocks, int iters, unsigned long long* clocks, void* stream);

/* Whether MFMAs and vector-ALU instructions overlap.  `blocks` workgroups of
 * eight waves, one per compute unit at a time (each holds 96 KB of LDS), so
 * each SIMD holds two of a workgroup's waves.  Per iteration, "MFMA work" is
 * 32 independent v_mfma_f32_16x16x32_bf16 and "vector work" 32 FMAs, 32
 * exp2, 16 bf16 packs and 16 XORs (the fine kernel's vector mix per 64-key
 * chunk and wave).  mode 0: every wave does `iters` iterations of MFMA work;
 * 1: of vector work; 2: waves 0-3 MFMA work and waves 4-7 vector work;
 * 3: every wave both, interleaved; 4: every wave the arithmetic of one
 * 64-key chunk of the fine kernel per iteration (S^T = K Q^T for two 16-query
 * sub-tiles, the bf16 weights, the all-ones denominators, O^T += V^T P^T:
 * 36 MFMAs, 32 FMAs, 32 exp2, 16 packs) with its K and V^T operands read
 * from LDS as the fine kernel reads them; 5: the same with the operands in
 * registers.  `clocks` (may be NULL): uint64
 * [blocks][8], each wave's elapsed shader clocks; `simd` (may be NULL, used
 * only with clocks): int32 [blocks][8], each wave's SIMD (HW_ID bits 5:4).
 * `sink` (float32 [blocks]) as above.  hipErrorInvalidValue for a mode
 * outside 0..5. */
int mosaic_probe_overlap(float* sink, int blocks, int iters, int mode, unsigned long long* clocks, int* simd,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOSAIC_PROBE_H */
