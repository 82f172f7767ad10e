// Fine attention: selected-block branch + sliding-window branch + gated sum.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse
// Attention: (b) every query of block i attends at full resolution to the
// tokens of the key blocks chosen for block i (one selection per block, as
// also stated in the mlsanity.com abstract and the paper-curation page's
// "How" section); (c) every query attends to a sliding window of nearby
// NESTED tokens; out = g_CG·o_CG + g_FG·o_FG + g_L·o_L.  The window is taken
// centred, [t - floor(W/2), t + ceil(W/2)) clipped to [0, N), and the
// selected branch is one softmax over the union of the selected tokens.
//
// Design (gfx950, wave64):
//   * one workgroup = 64 consecutive queries of one slice, 4 waves x 16
//     queries; each wave keeps its 16 queries' q in registers.
//   * keys stream through LDS 64 at a time, K and V both row-major [key][d]
//     (16-byte writes).  The V^T operand of the P·V MFMA is read with the
//     gfx950 transposing LDS load ds_read_b64_tr_b16: within each group of 16
//     lanes, output lane i receives element i%4 of the 8-byte rows addressed by
//     source lanes 4j + i/4 (j = 0..3), so a source lane r of group g points
//     at key 32*jj + 16*h + 4*g + r/4, column 16*dt + 4*(r%4), and every lane
//     ends up with 4 keys of one head-dim column.  All four waves share each
//     staged chunk.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 keys x 16 queries per
//     tile); in that layout each lane owns 16 scores of one query, so the
//     online softmax (running max, exp2 with log2(e)/sqrt(d) folded in)
//     needs only two cross-lane steps per chunk, and the bf16-rounded weights
//     are already the B operand of O^T += V^T P^T; the denominator is the
//     same MFMA with an all-ones A operand (sum of the rounded weights).
//   * selected branch: the chunk gathers n*block tokens by the selection
//     indices (virtual key v -> token sel[v/block]*block + v%block); for
//     blocks smaller than 64 the tile's 64/block query blocks are taken in
//     turn, each by the wave(s) whose queries it holds.
//   * local branch: the union of the tile's windows is streamed; chunks
//     inside every window of a wave's 16 queries run unmasked, chunks outside
//     them are skipped, the rest are masked per score.
//   * epilogue: out = g0·o_CG[t/block] + g1·o_FG + g2·o_L, float32.
// Roofline: bf16 matrix work 4*d*(n*block + W) per query, HBM traffic at
// least q, k, v once plus gates, o_CG and out.
#include "bsa_common.h"

#include <math.h>

namespace mosaic {
namespace {

struct FineArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gates;
  const float* o_cg;
  const int32_t* sel;
  float* out;
  int n_tok;
  int block;
  int topn;
  int window;
  int m;
  int tiles;
  float scale_log2;   // log2(e) / sqrt(d)
};


struct SoftmaxState {
  float m;      // running max of raw scores (this lane's query)
  floatx4 l;    // running denominator of this lane's query (all four entries equal)
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// transposing 8-byte LDS read (ds_read_b64_tr_b16)
__device__ __forceinline__ shortx4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

template <int D>
struct Tile {
  static constexpr int KK = D / 32;   // bf16 k-steps over d for S = K Q^T
  static constexpr int DT = D / 16;   // 16-row tiles of O^T over d
  static constexpr int KROW = D + 8;  // padded K / V row (bf16 elements)
};

// Stage 64 keys into LDS.  token_of(kappa) returns the token index or -1.
template <int D, typename F>
__device__ __forceinline__ void stage_chunk(uint16_t* Ks, uint16_t* Vs, const uint16_t* kslice,
                                            const uint16_t* vslice, F token_of) {
  constexpr int KROW = Tile<D>::KROW;
  for (int p = threadIdx.x; p < 64 * (D / 8); p += 256) {
    const int kappa = p / (D / 8), e8 = p % (D / 8);
    const int tok = token_of(kappa);
    uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
    if (tok >= 0) {
      kx = *reinterpret_cast<const uint4*>(kslice + (size_t)tok * D + 8 * e8);
      vx = *reinterpret_cast<const uint4*>(vslice + (size_t)tok * D + 8 * e8);
    }
    *reinterpret_cast<uint4*>(Ks + kappa * KROW + 8 * e8) = kx;
    *reinterpret_cast<uint4*>(Vs + kappa * KROW + 8 * e8) = vx;
  }
}

// One 64-key chunk for this wave's 16 queries.  valid(kappa_index) decides
// per score when `masked`.
template <int D, typename V>
__device__ __forceinline__ void attend_chunk(const uint16_t* Ks, const uint16_t* Vs,
                                             const bf16x8 (&qf)[Tile<D>::KK],
                                             floatx4 (&o)[Tile<D>::DT], SoftmaxState& st,
                                             float c, bool masked, V valid) {
  constexpr int KK = Tile<D>::KK, DT = Tile<D>::DT, KROW = Tile<D>::KROW;
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, lg = lane / 16;

  float s[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (kt * 16 + lr) * KROW + 32 * kk + 8 * lg);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[kt][i] = acc[i];
  }
  if (masked) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!valid(16 * kt + 4 * lg + i)) s[kt][i] = -INFINITY;
  }

  float mx = s[0][0];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float msc = m_new == -INFINITY ? 0.f : m_new * c;
  const float alpha = __builtin_amdgcn_exp2f(st.m * c - msc);

  bf16x8 pb[2];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pb[kt >> 1][4 * (kt & 1) + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[kt][i], c, -msc)));
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
  // The denominator is the sum of the same bf16-rounded weights that multiply
  // V (an all-ones A operand), so each output is an exact convex combination
  // of the weights actually used; every row of that tile holds the sum.
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    st.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[j], st.l, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      // A operand V^T[d = 16*dt + lr][k-slots 8*lg + e]: key of slot e is
      // 32*j + 16*(e/4) + 4*lg + e%4, matching the score layout of pb[j]
      const uint16_t* src = Vs + (32 * j + 4 * lg + (lr >> 2)) * KROW + dt * 16 + 4 * (lr & 3);
      const shortx4 lo = lds_read_tr16(src);
      const shortx4 hi = lds_read_tr16(src + 16 * KROW);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[j], o[dt], 0, 0, 0);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void fine_kernel(FineArgs a) {
  constexpr int KK = Tile<D>::KK, DT = Tile<D>::DT, KROW = Tile<D>::KROW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * KROW];

  const int N = a.n_tok, B = a.block, n = a.topn, m = a.m;
  const long long slice = blockIdx.x / a.tiles;
  const int t0 = (blockIdx.x % a.tiles) * 64;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int tw = t0 + 16 * w;   // first query of this wave
  const int tq = tw + lr;       // this lane's query

  const size_t sbase = (size_t)slice * N * D;
  const uint16_t* qs = a.q + sbase;
  const uint16_t* ks = a.k + sbase;
  const uint16_t* vs = a.v + sbase;
  const float c = a.scale_log2;

  // B operand of S^T = K Q^T: Q[query lr][32*kk + 8*lg + e]
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qs + (size_t)tq * D + 32 * kk + 8 * lg);

  // ---- selected branch ------------------------------------------------
  floatx4 ofg[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) ofg[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  SoftmaxState sfg = {-INFINITY, floatx4{0.f, 0.f, 0.f, 0.f}};
  const int nB = n * B;
  const int groups = B >= 64 ? 1 : 64 / B;
  for (int gi = 0; gi < groups; ++gi) {
    const int blk = t0 / B + gi;
    const bool active = B >= 64 || tw / B == blk;
    const int32_t* selrow = a.sel + ((size_t)slice * m + blk) * n;
    for (int vc0 = 0; vc0 < nB; vc0 += 64) {
      __syncthreads();
      stage_chunk<D>(Ks, Vs, ks, vs, [&](int kappa) {
        const int vk = vc0 + kappa;
        if (vk >= nB) return -1;
        int j = selrow[vk / B];
        j = j < 0 ? 0 : (j >= m ? m - 1 : j);   // never read outside the slice
        return j * B + vk % B;
      });
      __syncthreads();
      if (active)
        attend_chunk<D>(Ks, Vs, qf, ofg, sfg, c, nB - vc0 < 64, [&](int kappa) { return vc0 + kappa < nB; });
    }
  }

  // ---- local branch -----------------------------------------------------
  floatx4 ol[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) ol[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  SoftmaxState sl = {-INFINITY, floatx4{0.f, 0.f, 0.f, 0.f}};
  const int lo_off = a.window / 2, hi_off = a.window - a.window / 2;
  const int wlo = max(0, t0 - lo_off);
  const int whi = (int)min((long long)N, (long long)t0 + 63 + hi_off);
  const int ulo = max(0, tw - lo_off);                                 // union of this wave's windows
  const int uhi = (int)min((long long)N, (long long)tw + 15 + hi_off);
  const int ilo = max(0, tw + 15 - lo_off);                            // intersection of them
  const int ihi = (int)min((long long)N, (long long)tw + hi_off);
  for (int u0 = wlo; u0 < whi; u0 += 64) {
    __syncthreads();
    stage_chunk<D>(Ks, Vs, ks, vs, [&](int kappa) { return u0 + kappa < whi ? u0 + kappa : -1; });
    __syncthreads();
    if (u0 < uhi && u0 + 64 > ulo) {
      const bool full = u0 >= ilo && u0 + 64 <= ihi;
      attend_chunk<D>(Ks, Vs, qf, ol, sl, c, !full, [&](int kappa) {
        const int u = u0 + kappa;
        return u >= tq - lo_off && u < tq + hi_off && u < N;
      });
    }
  }

  // ---- gated sum ----------------------------------------------------------
  const float lfg = sfg.l[0], ll = sl.l[0];
  const float* g = a.gates + ((size_t)slice * N + tq) * 3;
  const float g0 = g[0], g1 = g[1] / lfg, g2 = g[2] / ll;
  const float* ocg = a.o_cg + ((size_t)slice * m + tq / B) * D;
  float* dst = a.out + ((size_t)slice * N + tq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d0 = dt * 16 + 4 * lg;
    const float4 cg = *reinterpret_cast<const float4*>(ocg + d0);
    float4 r;
    r.x = g0 * cg.x + g1 * ofg[dt][0] + g2 * ol[dt][0];
    r.y = g0 * cg.y + g1 * ofg[dt][1] + g2 * ol[dt][1];
    r.z = g0 * cg.z + g1 * ofg[dt][2] + g2 * ol[dt][2];
    r.w = g0 * cg.w + g1 * ofg[dt][3] + g2 * ol[dt][3];
    *reinterpret_cast<float4*>(dst + d0) = r;
  }
}

}  // namespace

hipError_t launch_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gates,
                       const float* o_cg, const int32_t* sel, float* out, long long slices,
                       int n_tok, int head_dim, int block, int topn, int window,
                       hipStream_t stream) {
  FineArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gates = gates;
  a.o_cg = o_cg;
  a.sel = sel;
  a.out = out;
  a.n_tok = n_tok;
  a.block = block;
  a.topn = topn;
  a.window = window;
  a.m = n_tok / block;
  a.tiles = n_tok / 64;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  dim3 grid((unsigned)(slices * a.tiles));
  if (head_dim == 64)
    hipLaunchKernelGGL(fine_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fine_kernel<32>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mosaic
