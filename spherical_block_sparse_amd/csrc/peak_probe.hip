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
//   * mosaic_probe_overlap: whether MFMAs and vector instructions of two
//     waves on one SIMD, or of one wave, run at the same time (below).
// Each folds what it computed into one value per workgroup, written only
// when it equals a value it never takes, so the work cannot be dropped.
#include "mosaic_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

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

// MFMA / vector-ALU overlap.  A workgroup of eight waves holds a 96 KB LDS
// array, so one workgroup runs per compute unit and each SIMD holds two of
// its waves (the kernel records each wave's SIMD from HW_ID to confirm which
// two).  An iteration of "MFMA work" is 32 independent
// v_mfma_f32_16x16x32_bf16 (eight accumulators); an iteration of "vector
// work" is the fine kernel's per-chunk vector mix: 32 FMAs and 32 exp2 in
// eight independent chains, 16 bf16 packs of the exp2 results and 16 XORs
// that fold the packs into a checksum.  MODE 0: every wave does MFMA work;
// 1: every wave does vector work; 2: waves 0-3 MFMA work, waves 4-7 vector
// work; 3: every wave does both, a round of 8 MFMAs then a quarter of the
// vector work, four times per iteration.
constexpr int kOverlapLds = 96 * 1024;

template <int MODE>
__global__ __launch_bounds__(512) void probe_overlap_kernel(float* sink, int iters, unsigned long long* clocks,
                                                            int* simd) {
  __shared__ float pad[kOverlapLds / 4];
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const bool mf = MODE == 0 || MODE == 3 || (MODE == 2 && w < 4);
  const bool va = MODE == 1 || MODE == 3 || (MODE == 2 && w >= 4);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = static_cast<__bf16>((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  floatx4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -0.25f - 0.001f * (float)((threadIdx.x + j) & 15);
  uint32_t chk = 0;
  // a quarter of the vector work: 8 FMAs, 8 exp2, 4 packs, 4 XORs
  auto vround = [&]() __attribute__((always_inline)) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = fmaf(x[j], 0.5f, -0.25f);
      p[j] = __builtin_amdgcn_exp2f(x[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bf16x2 pk;
      pk[0] = static_cast<__bf16>(p[j]);
      pk[1] = static_cast<__bf16>(p[j + 1]);
      chk ^= __builtin_bit_cast(uint32_t, pk);
    }
  };
  auto mround = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  };
  if constexpr (MODE == 3) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mround();
        vround();
      }
  } else {
    if (mf)
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) mround();
    if (va)
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) vround();
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  pad[threadIdx.x] = s + (float)chk;
  __syncthreads();
  if (pad[(threadIdx.x + 64) % 512] == -1234.5f) sink[blockIdx.x] = s;
  if (clocks && threadIdx.x % 64 == 0) {
    clocks[(size_t)blockIdx.x * 8 + w] = __builtin_amdgcn_s_memtime() - t0;
    // HW_ID bits 5:4 hold the wave's SIMD (s_getreg_b32 size 2, offset 4, register 4)
    if (simd) simd[(size_t)blockIdx.x * 8 + w] = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
  }
}

// The attention chunk's arithmetic without its loads and barrier: per
// iteration a wave forms S^T = K Q^T for 64 keys and two 16-query sub-tiles
// (16 MFMAs), the weights exp2(S c - m) in bf16 (32 FMAs, 32 exp2, 16
// packs), the denominators with an all-ones operand (4 MFMAs) and
// O^T += V^T P^T (16 MFMAs), the dependency chain of a 64-key chunk of the
// fine kernel.  LDS: the K operands are read from a 64 x 64 bf16 tile in LDS
// (two such K/V tile pairs, alternating between iterations so that the reads
// stay inside the loop)
// (8 reads of 16 bytes per lane, rows XOR-swizzled in 16-byte pieces so that
// 16 consecutive rows hit distinct banks) and the V^T operands with the
// transposing 8-byte read (16 per lane), as the fine kernel reads them;
// otherwise the same operands come from registers.
template <bool LDS>
__global__ __launch_bounds__(512) void probe_chunk_kernel(float* sink, int iters, unsigned long long* clocks,
                                                          int* simd) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[kOverlapLds / 2];   // K tile, V tile, the rest padding
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
  for (int e = threadIdx.x; e < 4 * 64 * 64; e += 512)
    kv[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>((float)((e * 7) & 15) * 0.0625f - 0.5f));
  __syncthreads();
  auto swz = [](int row) { return 2 * ((row >> 1) & 3) + ((row >> 3) & 1); };
  bf16x8 qf[2][2], kr[4][2], vr[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][kk][e] = static_cast<__bf16>((float)((lane + e + s + kk) & 7) * 0.03125f);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kr[i][j][e] = static_cast<__bf16>((float)((lane * 3 + e + i) & 7) * 0.0625f);
        vr[j][i][e] = static_cast<__bf16>((float)((lane + 5 * e + j) & 7) * 0.0625f);
      }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
  floatx4 o[2][4], l[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    l[s] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c = 0.18033688f, mref = 4.0f;
  for (int it = 0; it < iters; ++it) {
    const uint16_t* K = kv + (it & 1) * (2 * 64 * 64);   // this iteration's K tile, its V tile after it
    const uint16_t* V = K + 64 * 64;
    floatx4 acc[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc[s][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = kt * 16 + lr;
        const bf16x8 ka = LDS ? *reinterpret_cast<const bf16x8*>(K + row * 64 + 8 * ((4 * kk + lg) ^ swz(row)))
                              : kr[kt][kk];
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[s][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s][kk], acc[s][kt], 0, 0, 0);
      }
    bf16x8 pb[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pb[s][kt >> 1][4 * (kt & 1) + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(acc[s][kt][i], c, -mref)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int s = 0; s < 2; ++s) l[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[s][j], l[s], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        bf16x8 va;
        if constexpr (LDS) {
          const int row = 32 * j + 4 * lg + (lr >> 2);
          const int col = dt * 16 + 4 * (lr & 3);
          const uint16_t* src = V + row * 64 + 8 * ((col >> 3) ^ swz(row)) + (col & 7);
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(src));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(src + 16 * 64));
          va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          va = vr[j][dt];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) o[s][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[s][j], o[s][dt], 0, 0, 0);
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    sum += l[s][0];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) sum += o[s][dt][0] + o[s][dt][1] + o[s][dt][2] + o[s][dt][3];
  }
  if (sum == -1234.5f || kv[(threadIdx.x * 97) % (kOverlapLds / 2)] == 0x7fc1) sink[blockIdx.x] = sum;
  if (clocks && lane == 0) {
    clocks[(size_t)blockIdx.x * 8 + w] = __builtin_amdgcn_s_memtime() - t0;
    if (simd) simd[(size_t)blockIdx.x * 8 + w] = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
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

int mosaic_probe_overlap(float* sink, int blocks, int iters, int mode, unsigned long long* clocks, int* simd,
                         void* stream) {
  if (!sink || blocks < 1 || iters < 1 || mode < 0 || mode > 5) return (int)hipErrorInvalidValue;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks), block(512);
  switch (mode) {
    case 0: hipLaunchKernelGGL(probe_overlap_kernel<0>, grid, block, 0, hs, sink, iters, clocks, simd); break;
    case 1: hipLaunchKernelGGL(probe_overlap_kernel<1>, grid, block, 0, hs, sink, iters, clocks, simd); break;
    case 2: hipLaunchKernelGGL(probe_overlap_kernel<2>, grid, block, 0, hs, sink, iters, clocks, simd); break;
    case 3: hipLaunchKernelGGL(probe_overlap_kernel<3>, grid, block, 0, hs, sink, iters, clocks, simd); break;
    case 4: hipLaunchKernelGGL(probe_chunk_kernel<true>, grid, block, 0, hs, sink, iters, clocks, simd); break;
    default: hipLaunchKernelGGL(probe_chunk_kernel<false>, grid, block, 0, hs, sink, iters, clocks, simd); break;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
