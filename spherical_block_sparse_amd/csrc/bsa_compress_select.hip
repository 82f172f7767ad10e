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
//     key blocks stream through LDS 64 at a time (k̄ float64, v̄ float32).
//   * logits transposed, S^T = K̄ Q̄^T, with v_mfma_f64_16x16x4_f64 on the
//     exact float64 block means: in that layout lane l owns 16 logits of row
//     l%16, which is also the B operand layout of O^T += V̄^T P^T
//     (v_mfma_f32_16x16x4_f32), so the online softmax (running max, exp2 in
//     float32) needs no LDS round trip and only two cross-lane steps.
//   * ranking uses the float64 dot products themselves (dividing by sqrt(d)
//     is monotone), so the selection equals a float64 evaluation up to the
//     summation order of 64 products.
//   * top-n: each row keeps its current n-th best (value, index) key; the
//     logits that beat it are appended to the row's LDS buffer with an LDS
//     atomic, and when a buffer passes 64 entries one wave compacts it to its
//     best n with a 128-element bitonic network (DPP / swizzle exchanges),
//     which raises the key.  A final compaction orders the n survivors.
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
  double c_exp2;   // log2(e) / sqrt(d): exp(s) = 2^(dot * c_exp2)
};

constexpr int kCap = 128;   // candidate buffer per row

// (value, index) order of the selection: larger value first, then lower index
__device__ __forceinline__ bool beats(double av, int ai, double bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// x from lane (lane ^ J)
template <int J>
__device__ __forceinline__ int xor_lane(int x) {
  if constexpr (J == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  else if constexpr (J == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  else if constexpr (J <= 16) return __builtin_amdgcn_ds_swizzle(x, (J << 10) | 0x1F);   // bit mode, xor J
  else return __builtin_amdgcn_ds_bpermute(((int)(threadIdx.x & 63) ^ J) << 2, x);
}

// compare-exchange of position p with p ^ J inside a bitonic block of size K
template <int J, int K>
__device__ __forceinline__ void bitonic_step(double& v, int& i, int p) {
  const long long b = __double_as_longlong(v);
  const int plo = xor_lane<J>((int)(b & 0xffffffffLL));
  const int phi = xor_lane<J>((int)(b >> 32));
  const int pi = xor_lane<J>(i);
  const double pv = __longlong_as_double(((long long)phi << 32) | (unsigned)plo);
  const bool lower = (p & J) == 0;
  const bool desc = (p & K) == 0;
  const bool mine = beats(v, i, pv, pi);
  if (!((lower == desc) ? mine : !mine)) {
    v = pv;
    i = pi;
  }
}

template <int K, int J>
__device__ __forceinline__ void bitonic_merge(double& v0, int& i0, double& v1, int& i1, int lane) {
  if constexpr (J == 64) {   // positions lane and lane+64 sit in the same lane
    if (!beats(v0, i0, v1, i1)) {
      const double tv = v0; const int ti = i0;
      v0 = v1; i0 = i1; v1 = tv; i1 = ti;
    }
  } else {
    bitonic_step<J, K>(v0, i0, lane);
    bitonic_step<J, K>(v1, i1, lane + 64);
  }
  if constexpr (J > 1) bitonic_merge<K, J / 2>(v0, i0, v1, i1, lane);
}

// Sort the 128 entries (position p = lane + 64*h) best first.
template <int K = 128>
__device__ __forceinline__ void bitonic_sort(double& v0, int& i0, double& v1, int& i1, int lane) {
  if constexpr (K > 2) bitonic_sort<K / 2>(v0, i0, v1, i1, lane);
  bitonic_merge<K, K / 2>(v0, i0, v1, i1, lane);
}

template <int D>
__global__ __launch_bounds__(256) void compress_select_kernel(CSArgs a) {
  constexpr int KS = D / 4;    // f64 MFMA k-steps over the head dimension
  constexpr int DT = D / 16;   // 16-row tiles of O^T over the head dimension
  __shared__ double Ks[64][D + 1];
  __shared__ float Vs[64][D + 16];
  __shared__ double BufV[64][kCap];
  __shared__ int BufI[64][kCap];
  __shared__ int Cnt[64];
  __shared__ double ThrV[64];
  __shared__ int ThrI[64];

  const int m = a.m;
  const int n = a.topn;
  const long long slice = blockIdx.x / a.row_tiles;
  const int tile = blockIdx.x % a.row_tiles;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // scalar: uniform branches
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16;   // this lane's row within the wave
  const int lg = lane / 16;   // lane group 0..3
  const int rw = tile * 64 + w * 16;
  const int brow = w * 16 + lr;   // this lane's row in the workgroup buffers

  const double* qb = a.qbar + (size_t)slice * m * D;
  const double* kb = a.kbar + (size_t)slice * m * D;
  const float* vb = a.vbar + (size_t)slice * m * D;

  if (threadIdx.x < 64) {
    Cnt[threadIdx.x] = 0;
    ThrV[threadIdx.x] = -INFINITY;
    ThrI[threadIdx.x] = 0x7fffffff;
  }

  // B operand of S^T = K̄ Q̄^T: q̄[rw + lr][4*ks + lg]
  double qa[KS];
  {
    const int row = rw + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = row < m ? qb[(size_t)row * D + 4 * ks + lg] : 0.0;
  }

  floatx4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  double m_run = -INFINITY;   // running max of row lr (dot products)
  float l_run = 0.f;          // this lane's part of the running denominator
  double thr_v = -INFINITY;   // current n-th best key of row lr
  int thr_i = 0x7fffffff;

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

    // dot products: acc[ct][i] = q̄[row lr] · k̄[c0 + 16*ct + 4*i + lg]
    doublex4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(Ks[ct * 16 + lr][4 * ks + lg], qa[ks], acc[ct], 0, 0, 0);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c0 + 16 * ct + 4 * i + lg >= m) acc[ct][i] = -INFINITY;

    // online softmax of row lr and O^T += V̄^T P^T
    double cmax = acc[0][0];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmax(cmax, acc[ct][i]);
    cmax = fmax(cmax, __shfl_xor(cmax, 16));
    cmax = fmax(cmax, __shfl_xor(cmax, 32));
    const double m_new = fmax(m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f((float)((m_run - m_new) * a.c_exp2));
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f((float)((acc[ct][i] - m_new) * a.c_exp2));
        l_run += p;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(Vs[16 * ct + 4 * i + lg][dt * 16 + lr], p, oacc[dt], 0, 0, 0);
      }
    m_run = m_new;

    // selection: append the logits that beat the row's current n-th key
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = c0 + 16 * ct + 4 * i + lg;
        const bool cand = col < m && beats(acc[ct][i], col, thr_v, thr_i);
        if (__ballot(cand)) {
          if (cand) {
            const int pos = atomicAdd(&Cnt[brow], 1);
            BufV[brow][pos] = acc[ct][i];
            BufI[brow][pos] = col;
          }
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // compact rows whose buffer passed 64 entries (the next chunk adds <= 64)
    for (int r = 0; r < 16; ++r) {
      const int R = w * 16 + r;
      const int c = Cnt[R];
      if (c <= 64) continue;
      double v0 = lane < c ? BufV[R][lane] : -INFINITY;
      int i0 = lane < c ? BufI[R][lane] : 0x7fffffff;
      double v1 = lane + 64 < c ? BufV[R][lane + 64] : -INFINITY;
      int i1 = lane + 64 < c ? BufI[R][lane + 64] : 0x7fffffff;
      bitonic_sort(v0, i0, v1, i1, lane);
      const double tv = __shfl(v0, n - 1);
      const int ti = __shfl(i0, n - 1);
      if (lane < n) {
        BufV[R][lane] = v0;
        BufI[R][lane] = i0;
      }
      if (lane == 0) {
        ThrV[R] = tv;
        ThrI[R] = ti;
        Cnt[R] = n;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    thr_v = ThrV[brow];
    thr_i = ThrI[brow];
  }

  // o_CG = O / l; lane l holds rows lr, head-dim entries dt*16 + 4*lg + i
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (rw + lr < m) {
    const float inv = 1.0f / l_run;
    float* dst = a.o_cg + ((size_t)slice * m + rw + lr) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + dt * 16 + 4 * lg) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
  }

  // final top-n of every row, written in ascending block order
  for (int r = 0; r < 16; ++r) {
    if (rw + r >= m) break;
    const int R = w * 16 + r;
    const int c = Cnt[R];
    double v0 = lane < c ? BufV[R][lane] : -INFINITY;
    int i0 = lane < c ? BufI[R][lane] : 0x7fffffff;
    double v1 = lane + 64 < c ? BufV[R][lane + 64] : -INFINITY;
    int i1 = lane + 64 < c ? BufI[R][lane + 64] : 0x7fffffff;
    bitonic_sort(v0, i0, v1, i1, lane);
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += __shfl(i0, j) < i0 ? 1 : 0;
    if (lane < n) a.sel[((size_t)slice * m + rw + r) * n + rank] = i0;
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
  a.c_exp2 = 1.4426950408889634 / sqrt((double)head_dim);
  dim3 grid((unsigned)(slices * a.row_tiles));
  if (head_dim == 64)
    hipLaunchKernelGGL(compress_select_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(compress_select_kernel<32>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mosaic
