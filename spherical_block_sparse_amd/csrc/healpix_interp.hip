// Lat-lon -> HEALPix cross-attention interpolation.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED: for each
// HEALPix target i, the relative positions p_ij of its neighbouring source
// points are the queries and the source features the keys and values,
// o_i = sum_{j in N_i} softmax_j(q_ij^T k_j / sqrt(d)) v_j, with q_ij a
// linear map W_q p_ij of the 3-vector p_ij (this library's reading).
//
// Since q_ij^T k_j = p_ij^T (W_q^T k_j), the scores need only the 3-vector
// kappa_j = W_q^T k_j / sqrt(d) of each source point, formed once:
//   * kappa_kernel: eight lanes per source row (a wave reads eight whole
//     rows), W_q in LDS, float32 dot products of the bf16 row summed across
//     the eight lanes; HBM-bound (d*2 bytes read, 16 written);
//   * interp_kernel: one 16-lane group per target.  Lane l holds neighbour l
//     (index, relative position, kappa -> score); max and sum over the group
//     by shuffles; then lane l accumulates 8 output dims over half of the
//     neighbours from 16-byte pieces (one load instruction brings two whole
//     128-byte v rows per group), and lanes l, l ^ 8 add their halves.  All
//     16 rows are in flight at once, issued as soon as the indices are
//     known.  Targets in NESTED order share most of
//     their stencils, so the gathered rows hit in L2; the workgroup order is
//     XCD-contiguous.  HBM-bound.
#include "bsa_common.h"

#include <math.h>

namespace mosaic {
namespace {

// rows handled by each 8-lane group: their loads are all issued before any
// is used, so a wave keeps kRowsPerGroup KB in flight (one 16-byte load per
// lane and row leaves the kernel latency-bound at about half of HBM peak)
constexpr int kRowsPerGroup = 4;

__global__ __launch_bounds__(256) void kappa_kernel(const uint16_t* k, const float* w_q, float4* kappa, long long rows,
                                                    int d, float inv_sqrt_d) {
  __shared__ float W[256 * 3];
  for (int e = threadIdx.x; e < 3 * d; e += 256) W[e] = w_q[e];
  __syncthreads();
  // 8 lanes per row, each taking 16-byte pieces 8*e, 8*e + 64, ... of it, so
  // a wave reads 8 consecutive rows as one contiguous span; the group's rows
  // are 32 apart, so each of its loads is one such span of its wave
  const long long row0 = (long long)blockIdx.x * 32 * kRowsPerGroup + threadIdx.x / 8;
  const int e = threadIdx.x % 8;
  for (int c0 = 0; c0 < d; c0 += 64) {   // d <= 64 in one pass; larger d in passes of 64
    const int c = c0 + 8 * e;
    uint4 u[kRowsPerGroup];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      const long long row = row0 + 32 * r;
      u[r] = row < rows && c < d ? *reinterpret_cast<const uint4*>(k + row * d + c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      const long long row = row0 + 32 * r;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f;
      const uint32_t w[4] = {u[r].x, u[r].y, u[r].z, u[r].w};
      if (c < d) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = __builtin_bit_cast(float, i & 1 ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
          const float* wr = W + 3 * (c + i);   // w_q[d][3], row c + i
          a0 = fmaf(wr[0], x, a0);
          a1 = fmaf(wr[1], x, a1);
          a2 = fmaf(wr[2], x, a2);
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        a0 += __shfl_xor(a0, o, 8);
        a1 += __shfl_xor(a1, o, 8);
        a2 += __shfl_xor(a2, o, 8);
      }
      if (row < rows && e == 0) {
        if (c0 == 0) {
          kappa[row] = make_float4(a0 * inv_sqrt_d, a1 * inv_sqrt_d, a2 * inv_sqrt_d, 0.f);
        } else {
          float4 t = kappa[row];
          t.x += a0 * inv_sqrt_d; t.y += a1 * inv_sqrt_d; t.z += a2 * inv_sqrt_d;
          kappa[row] = t;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void interp_kernel(const float4* kappa, const uint16_t* v, const int32_t* nbr,
                                                     const float* rel, float* out, long long groups, int n_src,
                                                     int n_dst, int n_nbr) {
  constexpr int DV = 64;
  long long logical;
  {
    const long long g = gridDim.x, b = blockIdx.x, q8 = g / 8, r8 = g % 8, xcd = b % 8, kq = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + kq : r8 * (q8 + 1) + (xcd - r8) * q8 + kq;
  }
  const long long item = logical * 16 + threadIdx.x / 16;   // (slice, target)
  if (item >= groups) return;                                // whole 16-lane groups leave together
  const long long s = item / n_dst;
  const int i = (int)(item - s * n_dst);
  const int l = threadIdx.x % 16;

  int j = 0;
  if (l < n_nbr) {
    j = nbr[(long long)i * n_nbr + l];
    j = j < 0 ? 0 : (j >= n_src ? n_src - 1 : j);
  }
  // the 16 value rows depend only on the indices: they are all issued before
  // the scores are formed, so their latency overlaps the kappa gather (a
  // lane past n_nbr has index 0 and, below, weight 0).  Lane l reads 16-byte
  // pieces 8*(l%8) .. +7 of rows 2*i + l/8: one load instruction brings two
  // whole 128-byte rows per group.
  const int h = l >> 3, c8 = 8 * (l & 7);
  const uint16_t* vs = v + s * (long long)n_src * DV + c8;
  uint4 rows[8];
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) rows[ii] = *reinterpret_cast<const uint4*>(vs + (long long)__shfl(j, 2 * ii + h, 16) * DV);

  float score = -INFINITY;
  if (l < n_nbr) {
    const float* p = rel + ((long long)i * n_nbr + l) * 3;
    const float4 kp = kappa[s * n_src + j];
    score = p[0] * kp.x + p[1] * kp.y + p[2] * kp.z;
  }
  float mx = score;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
  const float e = l < n_nbr ? __expf(score - mx) : 0.f;
  float sum = e;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 16);
  const float pw = e / sum;

  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const float pj = __shfl(pw, 2 * ii + h, 16);
    const uint32_t wv[4] = {rows[ii].x, rows[ii].y, rows[ii].z, rows[ii].w};
#pragma unroll
    for (int q = 0; q < 8; ++q)
      acc[q] = fmaf(pj, __builtin_bit_cast(float, q & 1 ? (wv[q / 2] & 0xffff0000u) : (wv[q / 2] << 16)), acc[q]);
  }
  // lanes l and l ^ 8 hold the two halves of the rows for the same 8 dims:
  // lane l keeps dims c8 + 4h .. +3 of the sum
  float4 o4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float mine = acc[4 * h + q], other = __shfl_xor(acc[4 * (1 - h) + q], 8, 16);
    (&o4.x)[q] = mine + other;
  }
  *reinterpret_cast<float4*>(out + item * DV + c8 + 4 * h) = o4;
}

}  // namespace

hipError_t launch_interp(const uint16_t* k, const uint16_t* v, const float* w_q, const int32_t* nbr,
                         const float* rel, long long slices, int n_src, int n_dst, int n_nbr, int d, float* out,
                         float4* kappa, hipStream_t stream) {
  const long long rows = slices * n_src;
  hipLaunchKernelGGL(kappa_kernel, dim3((unsigned)((rows + 32 * kRowsPerGroup - 1) / (32 * kRowsPerGroup))), dim3(256),
                     0, stream, k, w_q, kappa, rows, d, (float)(1.0 / sqrt((double)d)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long groups = slices * n_dst;
  hipLaunchKernelGGL(interp_kernel, dim3((unsigned)((groups + 15) / 16)), dim3(256), 0, stream, kappa, v, nbr, rel,
                     out, groups, n_src, n_dst, n_nbr);
  return hipGetLastError();
}

}  // namespace mosaic
