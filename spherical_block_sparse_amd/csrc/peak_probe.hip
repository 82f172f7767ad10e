// Measured ceilings of the GPU, reported beside the published peaks.
//
// Not part of the attention method: two probes that show what this GPU
// sustains on the two resources the BSA kernels are bound by, so that a
// kernel's fraction of the published peak can be read against what a
// kernel doing nothing else reaches.
//   * mosaic_probe_read: a streaming read of a device buffer, 16-byte
//     nontemporal loads, eight in flight per lane, consecutive workgroups on
//     consecutive 4 KB spans (the access pattern of the pooling kernel,
//     without its arithmetic).
//   * mosaic_probe_mfma: back-to-back v_mfma_f32_16x16x32_bf16 on register
//     operands, eight independent accumulators per wave (no loads at all);
//     optionally each workgroup's shader clocks (s_memtime) and 100 MHz
//     ticks (s_memrealtime) over its run, which give the clock it ran at.
// Each folds what it computed into one value per workgroup, written only
// when it equals a value it never takes, so the work cannot be dropped.
#include "mosaic_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* p, size_t n16, float* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x7f8badc0u) sink[blockIdx.x] = __uint_as_float(acc);
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(float* sink, int iters, unsigned long long* clocks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  floatx4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == -1234.5f) sink[blockIdx.x] = s;
  if (clocks && threadIdx.x == 0) {   // shader clocks and 100 MHz ticks of wave 0's run
    clocks[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
    clocks[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

extern "C" {

int mosaic_probe_read(const void* buf, size_t bytes, float* sink, int blocks, void* stream) {
  if (!buf || !sink) return (int)hipErrorInvalidValue;
  if (blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

int mosaic_probe_mfma(float* sink, int blocks, int iters, unsigned long long* clocks, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     sink, iters, clocks);
  return (int)hipGetLastError();
}

}  // extern "C"
