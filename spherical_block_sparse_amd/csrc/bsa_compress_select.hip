// Compressed branch + top-n block selection.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse
// Attention: block-level logits s_ij = q̄_i·k̄_j / sqrt(d_k), their row softmax
// gives the coarse block-to-block attention (o_CG_i = sum_j ā_ij v̄_j), and
// the same scores pick the top-n key blocks each query block attends to at
// full resolution.  Ties go to the lower block index; the chosen indices are
// written in ascending order.
//
// Design (gfx950):
//   * one workgroup = 64 query-block rows of one slice, 4 waves x 16 rows;
//     the key blocks stream through LDS 64 at a time (k̄ in float64, v̄ in
//     float32).
//   * logits: v_mfma_f64_16x16x4_f64 on the exact float64 block means, so
//     the ranking equals a float64 evaluation up to summation order (a few
//     ulps), far below any gap that decides a selection.
//   * softmax numerator/denominator: online (running max), p = 2^((s-max)
//     log2 e) in float32; o_CG += P·V̄ with v_mfma_f32_16x16x4_f32.
//   * top-n: per row a sorted list held one entry per lane (n <= 64);
//     each 64-key chunk is filtered against the current n-th entry with one
//     ballot, and only the survivors are inserted (shift by one lane).
// Roofline: float64 matrix work 2*m^2*d per slice for the logits plus
// float32 matrix work 2*m^2*d for ā·v̄; HBM traffic is only the pooled
// tensors, o_CG and the indices.
#include "bsa_common.h"

#include <math.h>

namespace mosaic {
namespace {

struct CSArgs {
  const double* qbar;
  const double* kbar;
  const float* vbar;
  float* o_cg;
  int32_t* sel;
  int m;
  int topn;
  int row_tiles;
  double sqrt_d;
};

constexpr double kLog2e = 1.4426950408889634;

__device__ __forceinline__ bool beats(double av, int ai, double bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int D>
__global__ __launch_bounds__(256) void compress_select_kernel(CSArgs a) {
  constexpr int KS = D / 4;    // f64 MFMA k-steps over the head dimension
  constexpr int DT = D / 16;   // 16-wide output tiles over the head dimension
  __shared__ double Ks[64][D + 1];
  __shared__ float Vs[64][D + 16];
  __shared__ double Ss[4][16][65];

  const int m = a.m;
  const long long slice = blockIdx.x / a.row_tiles;
  const int tile = blockIdx.x % a.row_tiles;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16;   // row (A operand) / column (B operand) within a tile
  const int lg = lane / 16;   // lane group 0..3
  const int rw = tile * 64 + w * 16;   // first row of this wave

  const double* qb = a.qbar + (size_t)slice * m * D;
  const double* kb = a.kbar + (size_t)slice * m * D;
  const float* vb = a.vbar + (size_t)slice * m * D;

  // A operand of the logit MFMA: q̄[rw + lr][4*ks + lg]
  double qa[KS];
  {
    const int row = rw + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = row < m ? qb[(size_t)row * D + 4 * ks + lg] : 0.0;
  }

  floatx4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  double m_run = -INFINITY;   // running max of row lr
  float l_run = 0.f;          // this lane's part of the running denominator of row lr

  // top-n lists: row r of this wave, entry `lane`, sorted best first
  double lv[16];
  int li[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    lv[r] = -INFINITY;
    li[r] = 0x7fffffff;
  }
  const int n = a.topn;

  for (int c0 = 0; c0 < m; c0 += 64) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * D / 2; idx += 256) {
      const int key = idx / (D / 2), pr = idx % (D / 2);
      double2 x = make_double2(0.0, 0.0);
      if (c0 + key < m) x = *reinterpret_cast<const double2*>(kb + (size_t)(c0 + key) * D + 2 * pr);
      Ks[key][2 * pr] = x.x;
      Ks[key][2 * pr + 1] = x.y;
    }
    for (int idx = threadIdx.x; idx < 64 * D / 4; idx += 256) {
      const int key = idx / (D / 4), qd = idx % (D / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + key < m) x = *reinterpret_cast<const float4*>(vb + (size_t)(c0 + key) * D + 4 * qd);
      *reinterpret_cast<float4*>(&Vs[key][4 * qd]) = x;
    }
    __syncthreads();

    // logits of this wave's 16 rows x 64 key blocks
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      doublex4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], Ks[ct * 16 + lr][4 * ks + lg], acc, 0, 0, 0);
      const int col = ct * 16 + lr;
      const bool ok = c0 + col < m;
#pragma unroll
      for (int i = 0; i < 4; ++i) Ss[w][4 * i + lg][col] = ok ? acc[i] / a.sqrt_d : -INFINITY;
    }
    __syncthreads();

    // online softmax over this chunk, row lr
    double cmax = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) cmax = fmax(cmax, Ss[w][lr][4 * kk + lg]);
    cmax = fmax(cmax, __shfl_xor(cmax, 16));
    cmax = fmax(cmax, __shfl_xor(cmax, 32));
    const double m_new = fmax(m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f((float)((m_run - m_new) * kLog2e));
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ar = __shfl(alpha, 4 * lg + i);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][i] *= ar;
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float p = __builtin_amdgcn_exp2f((float)((Ss[w][lr][4 * kk + lg] - m_new) * kLog2e));
      l_run += p;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p, Vs[4 * kk + lg][dt * 16 + lr], oacc[dt], 0, 0, 0);
    }
    m_run = m_new;

    // top-n: merge this chunk into each row's list
    const int col = c0 + lane;
    const bool valid_col = col < m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (rw + r >= m) break;   // uniform across the wave
      const double sv = Ss[w][r][lane];
      double wv = __shfl(lv[r], n - 1);
      int wi = __shfl(li[r], n - 1);
      unsigned long long mask = __ballot(valid_col && beats(sv, col, wv, wi));
      while (mask) {
        const int b = __ffsll((long long)mask) - 1;
        mask &= mask - 1;
        const double cv = __shfl(sv, b);
        const int ci = c0 + b;
        if (!beats(cv, ci, wv, wi)) continue;
        const int pos = __popcll(__ballot(lane < n && beats(lv[r], li[r], cv, ci)));
        const double upv = __shfl_up(lv[r], 1);
        const int upi = __shfl_up(li[r], 1);
        if (lane == pos) {
          lv[r] = cv;
          li[r] = ci;
        } else if (lane > pos && lane < n) {
          lv[r] = upv;
          li[r] = upi;
        }
        wv = __shfl(lv[r], n - 1);
        wi = __shfl(li[r], n - 1);
      }
    }
  }

  // finalize o_CG = O / l
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rw + 4 * lg + i;
    const float inv = 1.0f / __shfl(l_run, 4 * lg + i);
    if (row < m) {
      float* dst = a.o_cg + ((size_t)slice * m + row) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dst[dt * 16 + lr] = oacc[dt][i] * inv;
    }
  }

  // selected indices, ascending
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (rw + r >= m) break;
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += __shfl(li[r], j) < li[r] ? 1 : 0;
    if (lane < n) a.sel[((size_t)slice * m + rw + r) * n + rank] = li[r];
  }
}

}  // namespace

hipError_t launch_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                  float* o_cg, int32_t* sel, long long slices, int m, int head_dim,
                                  int topn, hipStream_t stream) {
  CSArgs a;
  a.qbar = qbar;
  a.kbar = kbar;
  a.vbar = vbar;
  a.o_cg = o_cg;
  a.sel = sel;
  a.m = m;
  a.topn = topn;
  a.row_tiles = (m + 63) / 64;
  a.sqrt_d = sqrt((double)head_dim);
  dim3 grid((unsigned)(slices * a.row_tiles));
  if (head_dim == 64)
    hipLaunchKernelGGL(compress_select_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(compress_select_kernel<32>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mosaic
