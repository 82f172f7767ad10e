// HEALPix NESTED coarsening of a field from Nside to Nside / 2^levels.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED: in
// NESTED order the children of pixel p are 4p .. 4p+3, so the 4^levels
// descendants of a coarse pixel are one contiguous run of rows; the notes'
// encoder downsamples its native-resolution field to a coarser HEALPix grid.
// The coarse value is taken as the mean of the descendants (the same reading
// as the BSA block pooling).
//
// Design: HBM-bound streaming.  One thread per (coarse pixel, 8-channel
// group): consecutive threads cover consecutive 16-byte pieces of the same
// rows, so every wave reads whole rows; the 4^levels rows of a coarse pixel
// are summed in float64 four at a time (independent loads in flight) and the
// mean is written as float32.  Bytes per coarse pixel: 2*C*4^levels read,
// 4*C written.
#include "bsa_common.h"

namespace mosaic {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void add_bf16x8(double (&acc)[8], u32x4 v) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += (double)__builtin_bit_cast(float, w[i] << 16);
    acc[2 * i + 1] += (double)__builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(256) void coarsen_kernel(const uint16_t* x, float* y, long long out_rows, int groups8,
                                                      int channels, int rows_per) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= out_rows * groups8) return;
  const long long orow = gid / groups8;
  const int c8 = (int)(gid - orow * groups8);
  const uint16_t* src = x + (orow * rows_per) * channels + 8 * c8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r = 0;
  for (; r + 4 <= rows_per; r += 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (long long)(r + u) * channels));
#pragma unroll
    for (int u = 0; u < 4; ++u) add_bf16x8(acc, v[u]);
  }
  for (; r < rows_per; ++r) add_bf16x8(acc, *reinterpret_cast<const u32x4*>(src + (long long)r * channels));
  const double inv = 1.0 / rows_per;
  float* dst = y + orow * channels + 8 * c8;
  *reinterpret_cast<float4*>(dst) = make_float4((float)(acc[0] * inv), (float)(acc[1] * inv),
                                                (float)(acc[2] * inv), (float)(acc[3] * inv));
  *reinterpret_cast<float4*>(dst + 4) = make_float4((float)(acc[4] * inv), (float)(acc[5] * inv),
                                                    (float)(acc[6] * inv), (float)(acc[7] * inv));
}

}  // namespace

hipError_t launch_coarsen(const uint16_t* x, float* y, long long batch, int n_tok, int channels, int levels,
                          hipStream_t stream) {
  const int rows_per = 1 << (2 * levels);
  const long long out_rows = batch * (n_tok / rows_per);
  const int groups8 = channels / 8;
  const long long threads = out_rows * groups8;
  hipLaunchKernelGGL(coarsen_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, y, out_rows,
                     groups8, channels, rows_per);
  return hipGetLastError();
}

}  // namespace mosaic
