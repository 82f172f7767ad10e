// Compressed branch + top-n block selection.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse
// Attention: block-level logits s_ij = q̄_i·k̄_j / sqrt(d_k), their row softmax
// gives the coarse block-to-block attention (o_CG_i = sum_j ā_ij v̄_j), and
// the same scores pick the top-n key blocks each query block attends to at
// full resolution.  Ties go to the lower block index; the chosen indices are
// written in ascending order.
//
// Kernels: with the pool's bf16 pieces of k̄ and n <= 16 (the forward's
// path), compress_select_apx_kernel ranks on approximate logits and
// certifies every row (its own section below), handing tiles it cannot
// settle to the float64 list kernel; otherwise the float64 kernels below
// run alone (list n <= 16, buffered n <= 64, generic any n).
//
// Design of the float64 kernels (gfx950):
//   * one workgroup = 64 query-block rows of one slice, 4 waves x 16 rows;
//     key blocks stream through LDS 32 at a time (k̄ float64, v̄ float32)
//     with direct global->LDS loads, double-buffered.
//   * logits transposed, S^T = K̄ Q̄^T, with v_mfma_f64_16x16x4_f64 on the
//     exact float64 block means: in that layout lane l owns 8 logits of row
//     l%16 per chunk (the keys congruent to l/16 mod 4), which is also the B
//     operand layout of O^T += V̄^T P^T (v_mfma_f32_16x16x32_bf16 on
//     bf16-rounded weights and v̄, with its k-slots permuted to match), so the
//     online softmax needs no LDS round trip and only two cross-lane steps.
//   * ranking uses the float64 dot products themselves (dividing by sqrt(d)
//     is monotone), so the selection equals a float64 evaluation up to the
//     summation order of the products.
//   * top-n, n <= 16 (list kernel): every lane keeps the best K >= n
//     (value, index) pairs of its own keys in registers (K = 8 or 16),
//     updated by a branch-free insertion; keys arrive in increasing index
//     order, so a strict compare settles ties.  A lane holds at most n of
//     the row's top n, so the union of the row's four lists contains them.
//     The insertion of a chunk position is skipped for the whole wave when
//     no lane's key beats its list's last entry and a lower bound of its
//     row's n-th best (the smallest of the four lanes' ceil(n/4)-th entries):
//     the 16 rows of a wave are neighbouring blocks that want largely the
//     same keys, so most positions are skipped.  The four lists are merged
//     in registers (two bitonic merges across lanes 16 and 32 apart) and the
//     n winners are sorted by block index.
//   * any n > 64: compress_select_generic_kernel, one wave per row with an
//     exact radix selection (below).
//   * buffered kernel (16 < n <= 64): each row keeps
//     its current n-th best key; logits that beat it are appended to an LDS
//     candidate buffer at prefix-count slots, and a buffer that could
//     overflow is compacted to its best n by a 128-entry bitonic network over
//     four rows at once (register and DPP / swizzle exchanges).
// Roofline: float64 matrix work 2*m^2*d per slice for the logits plus bf16
// matrix work 2*m^2*d for ā·v̄ (the approximate kernel: three bf16 products
// of 2*m^2*d for the logits); HBM traffic is only the pooled tensors, o_CG
// and the indices.
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
  int redo;        // list kernel only: recompute just the row tiles holding a row marked -1
  const uint16_t* kpieces;   // approximate kernel: bf16 pieces of k̄ [slices][m][2][D]
  const float* kbn2;         // approximate kernel: |k̄_j|^2 [slices][m]
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

// Four rows at once, one per 16-lane group: lane l of a group holds
// positions 8*l .. 8*l+7 of its row's 128-entry buffer in v[e], ix[e].
// Bitonic sort, best first.  Exchanges at distances 1, 2, 4 stay inside a
// lane (register compare-exchanges); distances 8 .. 64 are lane distances
// 1 .. 8 inside the 16-lane group (DPP / swizzle).
template <int J>
__device__ __forceinline__ void sort_lane_stage(double (&v)[8], int (&ix)[8], int l, int k) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e & J) continue;
    const int p = 8 * l + e;
    const bool desc = (p & k) == 0;
    const bool b = beats(v[e], ix[e], v[e | J], ix[e | J]);
    if (desc ? !b : b) {
      const double tv = v[e]; const int ti = ix[e];
      v[e] = v[e | J]; ix[e] = ix[e | J];
      v[e | J] = tv; ix[e | J] = ti;
    }
  }
}

template <int LD>   // lane distance
__device__ __forceinline__ void sort_cross_stage(double (&v)[8], int (&ix)[8], int l, int k) {
  const bool lower = (l & LD) == 0;
  const bool desc = ((8 * l) & k) == 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const long long b = __double_as_longlong(v[e]);
    const int plo = xor_lane<LD>((int)(b & 0xffffffffLL));
    const int phi = xor_lane<LD>((int)(b >> 32));
    const int pi = xor_lane<LD>(ix[e]);
    const double pv = __longlong_as_double(((long long)phi << 32) | (unsigned)plo);
    const bool mine = beats(v[e], ix[e], pv, pi);
    if (!((lower == desc) ? mine : !mine)) {
      v[e] = pv;
      ix[e] = pi;
    }
  }
}

__device__ __forceinline__ void sort_rows4(double (&v)[8], int (&ix)[8], int l) {
#pragma unroll
  for (int k = 2; k <= 128; k <<= 1) {
    if (k >= 128) sort_cross_stage<8>(v, ix, l, k);
    if (k >= 64) sort_cross_stage<4>(v, ix, l, k);
    if (k >= 32) sort_cross_stage<2>(v, ix, l, k);
    if (k >= 16) sort_cross_stage<1>(v, ix, l, k);
    if (k >= 8) sort_lane_stage<4>(v, ix, l, k);
    if (k >= 4) sort_lane_stage<2>(v, ix, l, k);
    sort_lane_stage<1>(v, ix, l, k);
  }
}


// 16 zero bytes: the direct-load source of rows past the last key block
__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

constexpr int kCols = 32;   // key blocks per streamed chunk

// LDS layouts of one chunk (rows are key blocks, no padding, so a wave's
// 1 KB direct load fills whole rows); 16-byte chunks XOR-swizzled per row:
//   k̄: D float64 per row (D/2 chunks), chunk c of row r at c ^ (r & 15):
//       the 16 rows read at one head-dim index by an f64 MFMA hit 16
//       different chunks;
//   v̄: D float32 per row (D/4 chunks), chunk c of row r at c ^ 4*(r & 3):
//       the four rows read together by the P·V MFMA start in different banks.
template <int D>
__device__ __forceinline__ int kswz(int r) { return r & (D / 2 - 1) & 15; }
template <int D>
__device__ __forceinline__ int vswz(int r) { return (4 * (r & 3)) & (D / 4 - 1); }

// Loads of the kCols key blocks starting at c0 into LDS: lane l of a 1 KB
// load writes bytes 16*l.. of that span, i.e. physical chunk
// (1024*g + 16*l) % ROW / 16 of row (1024*g + 16*l) / ROW, which holds the
// logical chunk given by the row's swizzle.  A whole chunk goes through
// buffer loads (fixed per-lane offsets, the chunk start as a scalar
// offset); a chunk reaching past m reads zeros for the missing rows.  The
// loads are untracked by the compiler (see dma_buffer); the caller waits.
template <int D>
__device__ __forceinline__ void issue_chunk(int c0, double* kb, float* vb, const char* kbytes,
                                            const char* vbytes, int32x4 rk, int32x4 rv, bool use_rsrc,
                                            int m, int w, int lane) {
  constexpr int KROW = D * 8, VROW = D * 4;   // bytes per LDS row
  constexpr int KLOADS = kCols * KROW / 1024 / 4, VLOADS = kCols * VROW / 1024 / 4;   // 1 KB loads per wave
  static_assert(KLOADS >= 1 && VLOADS >= 1, "chunk split");
  const bool whole = use_rsrc && c0 + kCols <= m;
#pragma unroll
  for (int gg = 0; gg < KLOADS; ++gg) {
    const int g = w + 4 * gg;
    const int byte = 1024 * g + 16 * lane;
    const int r = byte / KROW, pc = (byte % KROW) / 16;
    const int off = r * KROW + 16 * (pc ^ kswz<D>(r));
    char* dst = reinterpret_cast<char*>(kb) + 1024 * g;
    if (whole) dma_buffer(dst, off, rk, c0 * KROW);
    else dma_global(dst, c0 + r < m ? (const void*)(kbytes + (size_t)c0 * KROW + off) : (const void*)&kZero16);
  }
#pragma unroll
  for (int gg = 0; gg < VLOADS; ++gg) {
    const int g = w + 4 * gg;
    const int byte = 1024 * g + 16 * lane;
    const int r = byte / VROW, pc = (byte % VROW) / 16;
    const int off = r * VROW + 16 * (pc ^ vswz<D>(r));
    char* dst = reinterpret_cast<char*>(vb) + 1024 * g;
    if (whole) dma_buffer(dst, off, rv, c0 * VROW);
    else dma_global(dst, c0 + r < m ? (const void*)(vbytes + (size_t)c0 * VROW + off) : (const void*)&kZero16);
  }
}

// Dot products of one staged chunk: acc[ct][i] = q̄[row lr] · k̄[c0 + 16*ct + 4*i + lg],
// -inf past the last key block.  qa is the B operand q̄[row lr][4*ks + lg].
template <int D>
__device__ __forceinline__ void chunk_logits(doublex4 (&acc)[2], const double* kb, const double (&qa)[D / 4],
                                             int c0, int m, int lr, int lg) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) acc[ct] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int r = ct * 16 + lr, k = 4 * ks + lg;   // A operand k̄[r][k]
      const double kv = kb[r * D + 2 * ((k >> 1) ^ kswz<D>(r)) + (k & 1)];
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(kv, qa[ks], acc[ct], 0, 0, 0);
    }
  if (c0 + kCols > m) {   // the last chunk may reach past the key blocks
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c0 + 16 * ct + 4 * i + lg >= m) acc[ct][i] = -INFINITY;
  }
}

// Online softmax of row lr over one chunk and O^T += V̄^T P^T.  m_run is the
// running maximum dot product, l_run this lane's part of the denominator.
// The weights are rounded to bf16 and multiply bf16-rounded v̄ in one
// v_mfma_f32_16x16x32_bf16 per 16 head-dim rows: k-slot 8*g + e of that
// product holds key 16*(e/4) + 4*(e%4) + g, which is exactly the key whose
// logit lane lr + 16*g holds in acc[e/4][e%4], so the weights need no
// exchange between lanes.  The denominator adds the rounded weights (pairwise,
// v_dot2 with ones), so o_CG is an exact convex combination of the v̄ rows as
// the product sees them.
template <int D>
__device__ __forceinline__ void chunk_softmax_pv(const doublex4 (&acc)[2], const float* vb, double c_exp2,
                                                 double lazy, double& m_run, float& l_run,
                                                 floatx4 (&oacc)[D / 16], int lr, int lg) {
  // The reference m_run moves only when a logit exceeds it by more than
  // 2^8 after scaling (weights stay <= 256).  Each lane checks its own 8
  // logits and the wave votes, so the row maxima across the four lanes of a
  // row are formed only when some reference moves (a scalar branch).
  double lmax = acc[0][0];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) lmax = fmax(lmax, acc[ct][i]);
  if (__ballot(lmax > m_run + lazy)) {
    double row = fmax(lmax, __shfl_xor(lmax, 16));
    row = fmax(row, __shfl_xor(row, 32));
    const double m_new = fmax(m_run, row);
    const float alpha = m_run == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((float)((m_run - m_new) * c_exp2));
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
  }
  const double nmc = -m_run * c_exp2;
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    pb[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f((float)fma(acc[e / 4][e % 4], c_exp2, nmc)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int e = 0; e < 8; e += 2) l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e], pb[e + 1]}, ones, l_run, false);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int col = dt * 16 + lr;   // A operand v̄^T[col][slot 8*lg + e]
    bf16x8 va;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 16 * (e / 4) + 4 * (e % 4) + lg;
      va[e] = static_cast<__bf16>(vb[r * D + 4 * ((col >> 2) ^ vswz<D>(r)) + (col & 3)]);
    }
    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[dt], 0, 0, 0);
  }
}

// o_CG = O / l for row `row`; lane l holds head-dim entries dt*16 + 4*lg + i
template <int D>
__device__ __forceinline__ void store_ocg(float* o_cg_row, const floatx4 (&oacc)[D / 16], float l_run, int lg,
                                          bool valid) {
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (valid) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(o_cg_row + dt * 16 + 4 * lg) =
          make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// List kernel, n <= K: per-lane register lists of the best K keys.

// Insert (x, xi) into the list sorted best first.  xi is larger than every
// index already in the list, so x beats entry j exactly when x > tv[j], and
// with c_j = (x > tv[j]) monotone in j the new entry j is
// max(tv[j], min(tv[j-1], x)); the indices follow the same choice.  A key
// that beats no entry leaves the list unchanged.
template <int K>
__device__ __forceinline__ void list_insert(double (&tv)[K], int (&ti)[K], double x, int xi) {
  bool c[K];
#pragma unroll
  for (int j = 0; j < K; ++j) c[j] = x > tv[j];
#pragma unroll
  for (int j = K - 1; j >= 1; --j) {
    tv[j] = fmax(tv[j], fmin(tv[j - 1], x));
    ti[j] = c[j - 1] ? ti[j - 1] : (c[j] ? xi : ti[j]);
  }
  tv[0] = fmax(tv[0], x);
  ti[0] = c[0] ? xi : ti[0];
}

// a <- the better of (a, b), b <- the other
__device__ __forceinline__ void order_pair(double& av, int& ai, double& bv, int& bi) {
  if (beats(bv, bi, av, ai)) {
    const double tv = av; const int t = ai;
    av = bv; ai = bi; bv = tv; bi = t;
  }
}

// Replace the list by the best K of its union with the list of lane
// (lane ^ X), sorted best first: the pairwise better of a[j] and b[K-1-j]
// holds the best K as a bitonic sequence, which K/2-to-1 merging sorts.
// Both lanes end with the same list.
template <int K, int X>
__device__ __forceinline__ void merge_lanes(double (&tv)[K], int (&ti)[K]) {
  double pv[K];
  int pi[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    pv[j] = __shfl_xor(tv[j], X);
    pi[j] = __shfl_xor(ti[j], X);
  }
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (beats(pv[K - 1 - j], pi[K - 1 - j], tv[j], ti[j])) {
      tv[j] = pv[K - 1 - j];
      ti[j] = pi[K - 1 - j];
    }
#pragma unroll
  for (int s = K / 2; s >= 1; s >>= 1)
#pragma unroll
    for (int j = 0; j < K; ++j)
      if ((j & s) == 0) order_pair(tv[j], ti[j], tv[j + s], ti[j + s]);
}

template <int D, int K>
__global__ __launch_bounds__(256) void compress_select_list_kernel(CSArgs a) {
  __shared__ __attribute__((aligned(16))) double Kb0[kCols * D];
  __shared__ __attribute__((aligned(16))) float Vb0[kCols * D];
  __shared__ __attribute__((aligned(16))) double Kb1[kCols * D];
  __shared__ __attribute__((aligned(16))) float Vb1[kCols * D];

  // contiguous run of row tiles per XCD (workgroups are dispatched
  // round-robin over the 8 XCDs): the tiles of one slice then read its k̄, v̄
  // through one L2
  long long logical;
  {
    const long long G = gridDim.x, b = blockIdx.x;
    const long long q8 = G / 8, r8 = G % 8, xcd = b % 8, k = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + k : r8 * (q8 + 1) + (xcd - r8) * q8 + k;
  }
  const int m = a.m;
  const int n = a.topn;
  const int jb = (n + 3) / 4 - 1;   // each lane's entry jb bounds its row's n-th best from below
  const long long slice = logical / a.row_tiles;
  const int tile = (int)(logical % a.row_tiles);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // scalar: uniform branches
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16;   // this lane's row within the wave
  const int lg = lane / 16;   // lane group 0..3: keys congruent to lg mod 4
  const int rw = tile * 64 + w * 16;
  const int row = rw + lr;
  if (a.redo) {   // only tiles in which the approximate pass left rows to this kernel
    const int r = tile * 64 + (int)threadIdx.x;
    const bool marked = threadIdx.x < 64 && r < m && a.sel[((size_t)slice * m + r) * n] < 0;
    if (!__syncthreads_or(marked)) return;
  }

  const double* qb = a.qbar + (size_t)slice * m * D;
  const char* kbytes = reinterpret_cast<const char*>(a.kbar + (size_t)slice * m * D);
  const char* vbytes = reinterpret_cast<const char*>(a.vbar + (size_t)slice * m * D);
  const bool use_rsrc = (long long)m * D * 8 < 0x7fffffffLL;   // 32-bit buffer offsets
  const int32x4 rk = slice_rsrc(kbytes, use_rsrc ? m * D * 8 : 0);
  const int32x4 rv = slice_rsrc(vbytes, use_rsrc ? m * D * 4 : 0);
  const double lazy = 8.0 / a.c_exp2;   // 2^8 in weight, in units of raw dot products

  double qa[D / 4];
#pragma unroll
  for (int ks = 0; ks < D / 4; ++ks) qa[ks] = row < m ? qb[(size_t)row * D + 4 * ks + lg] : 0.0;

  floatx4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  double m_run = -INFINITY;
  float l_run = 0.f;
  double tv[K];
  int ti[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    tv[j] = -INFINITY;
    ti[j] = 0x7fffffff;
  }

  auto chunk = [&](int c0, const double* kb, const float* vb) __attribute__((always_inline)) {
    doublex4 acc[2];
    chunk_logits<D>(acc, kb, qa, c0, m, lr, lg);
    chunk_softmax_pv<D>(acc, vb, a.c_exp2, lazy, m_run, l_run, oacc, lr, lg);
    // a key below `bound` is beaten by n keys of its row: never needed
    double bound = tv[0];
#pragma unroll
    for (int j = 1; j < K && j < 4; ++j)
      if (jb == j) bound = tv[j];
    bound = fmin(bound, __shfl_xor(bound, 16));
    bound = fmin(bound, __shfl_xor(bound, 32));
    // A key enters the list step when it reaches max(tv[K-1], bound).  That
    // admits, besides the keys with x > tv[K-1] and x >= bound, only
    // x == tv[K-1], which the strict compares of list_insert leave out.
    double thr = fmax(tv[K - 1], bound);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double x = acc[ct][i];
        if (__ballot(x >= thr)) {
          list_insert<K>(tv, ti, x, c0 + 16 * ct + 4 * i + lg);
          thr = fmax(tv[K - 1], bound);
        }
      }
  };

  issue_chunk<D>(0, Kb0, Vb0, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int c0 = 0; c0 < m; c0 += 2 * kCols) {
    if (c0 + kCols < m) issue_chunk<D>(c0 + kCols, Kb1, Vb1, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
    chunk(c0, Kb0, Vb0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (c0 + kCols >= m) break;
    if (c0 + 2 * kCols < m) issue_chunk<D>(c0 + 2 * kCols, Kb0, Vb0, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
    chunk(c0 + kCols, Kb1, Vb1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  store_ocg<D>(a.o_cg + ((size_t)slice * m + row) * D, oacc, l_run, lg, row < m);

  // best K of the row's four lists, in every lane of the row
  merge_lanes<K, 16>(tv, ti);
  merge_lanes<K, 32>(tv, ti);
  // the best n, by ascending block index (bitonic sort of K indices with the
  // entries past n set to INT_MAX); lane group lg writes entries
  // lg*K/4 .. lg*K/4 + K/4 - 1
  int ix[K];
#pragma unroll
  for (int j = 0; j < K; ++j) ix[j] = j < n ? ti[j] : 0x7fffffff;
#pragma unroll
  for (int k = 2; k <= K; k <<= 1)
#pragma unroll
    for (int s = k / 2; s >= 1; s >>= 1)
#pragma unroll
      for (int j = 0; j < K; ++j)
        if ((j & s) == 0) {
          const bool up = (j & k) == 0;
          const int lo = min(ix[j], ix[j + s]), hi = max(ix[j], ix[j + s]);
          ix[j] = up ? lo : hi;
          ix[j + s] = up ? hi : lo;
        }
  if (row < m) {
    int32_t* dst = a.sel + ((size_t)slice * m + row) * n;
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j / (K / 4) == lg && j < n) dst[j] = ix[j];
  }
}

// ---------------------------------------------------------------------------
// Approximate kernel, n <= 16: bf16-piece logits, then a certified selection.
//
// The float64 logits above cost 2·m²·d float64 matrix work, about half of
// this stage.  Only the order of each row's keys at its n-th/(n+1)-th
// boundary needs float64.  This kernel ranks with approximate logits and
// certifies the result:
//   * pieces: x = x1 + x2 + r with x1 = bf16(x), x2 = bf16(x - x1) and
//     |r| <= (2^-16 + 2^-24) |x|.  The pooling writes the pieces of k̄
//     ([m][2][d] bf16, natural channel order) and |k̄_j|^2 of every block;
//     q̄ is split here, in registers.  The logit s~ = q1·k1 + q1·k2 + q2·k1
//     takes 3 products per 32 of d on v_mfma_f32_16x16x32_bf16, whose
//     bf16 x bf16 products are exact in float32.  The dropped terms are below
//     3.1·2^-16 |q̄_c k̄_c| per channel and the float32 sum of the 3d products
//     errs by at most γ_{3d-1} = 191·2^-24 (d = 64) of the sum of their
//     magnitudes, twice that if the accumulator truncated; together under
//     2^-13.8 Σ_c |q̄_c k̄_c| <= 2^-13.8 |q̄| |k̄|.  The bound used is
//     ε_i = 2^-12.5 |q̄_i| max_j |k̄_j|, the maximum over the slice's key
//     blocks, read from the block norms before streaming.
//   * a chunk of 32 key blocks is 32 rows of pieces (4d bytes each) and 32
//     rows of v̄, staged by direct loads, double-buffered, one barrier per
//     chunk.  The MFMA's A rows are the chunk's keys in the order
//     4(m%4) + m/4, which leaves each logit in the lane and register where
//     the float64 kernel has it: the online softmax, ā·v̄ and the lane lists
//     are unchanged in structure (o_CG uses the approximate logits; its
//     weights are rounded to bf16 anyway).
//   * every key a lane's list lets go -- not inserted or evicted -- updates
//     the row's largest dropped value R.  Each lane lists its best 8 keys and
//     the merges keep all 32 of the row.  A row is certified when
//     R < s~_(n) - 2ε: every dropped key is then below the exact n-th logit.
//     Keys above s~_(n) + 2ε are in the top n, keys below s~_(n) - 2ε are
//     out, and the few in between are rescored in float64 (the same fused
//     multiply-adds for every key, so equal k̄ rows give equal values) and
//     ranked by (value, index).
//   * a row that fails (more than kBandMax keys in the band, or R inside
//     it: massive ties, or logits crowded closer than ε) is settled exactly
//     by the whole workgroup at the end: its float64 logits (cached in the
//     freed staging LDS when m <= 4096, else recomputed per pass), eight
//     8-bit radix passes for the n-th value and an ascending sweep
//     (exact_row).  A tile with more than kExactRows such rows is marked
//     instead (-1 as the rows' first index), and a second launch of the
//     float64 list kernel redoes the marked tiles; its other workgroups read
//     their tile's 64 marks and exit.
// A key more than 4ε below a lower bound of its row's n-th best is not
// inserted: it is below the final s~_(n) - 2ε, so it cannot fail the row.
constexpr double kApxEps = 1.7263349e-4;   // 2^-12.5
constexpr int kBandMax = 16;   // band entries rescored per row (list positions 16 .. 31 of the result)
// uncertified rows a workgroup settles itself; beyond that its tile is
// marked for the float64 list kernel
constexpr int kExactRows = 4;

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

template <int K>
__device__ __forceinline__ void list_insert_f(float (&tv)[K], int (&ti)[K], float x, int xi) {
  bool c[K];
#pragma unroll
  for (int j = 0; j < K; ++j) c[j] = x > tv[j];
#pragma unroll
  for (int j = K - 1; j >= 1; --j) {
    tv[j] = fmaxf(tv[j], fminf(tv[j - 1], x));
    ti[j] = c[j - 1] ? ti[j - 1] : (c[j] ? xi : ti[j]);
  }
  tv[0] = fmaxf(tv[0], x);
  ti[0] = c[0] ? xi : ti[0];
}

__device__ __forceinline__ bool beats_f(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ void order_pair_f(float& av, int& ai, float& bv, int& bi) {
  if (beats_f(bv, bi, av, ai)) {
    const float tv = av; const int t = ai;
    av = bv; ai = bi; bv = tv; bi = t;
  }
}

// bitonic merge of a length-L bitonic sequence into best-first order
template <int L>
__device__ __forceinline__ void bitonic_merge_f(float (&v)[L], int (&ix)[L]) {
#pragma unroll
  for (int s = L / 2; s >= 1; s >>= 1)
#pragma unroll
    for (int j = 0; j < L; ++j)
      if ((j & s) == 0) order_pair_f(v[j], ix[j], v[j + s], ix[j + s]);
}

// Float version of chunk_softmax_pv (same layout and rounding).
template <int D>
__device__ __forceinline__ void chunk_softmax_pv_f(const floatx4 (&acc)[2], const float* vb, float c, float lazy,
                                                   float& m_run, float& l_run, floatx4 (&oacc)[D / 16], int lr,
                                                   int lg) {
  float lmax = acc[0][0];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, acc[ct][i]);
  if (__ballot(lmax > m_run + lazy)) {
    float row = fmaxf(lmax, __shfl_xor(lmax, 16));
    row = fmaxf(row, __shfl_xor(row, 32));
    const float m_new = fmaxf(m_run, row);
    const float alpha = m_run == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
  }
  const float nmc = -m_run * c;
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(acc[e / 4][e % 4], c, nmc)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int e = 0; e < 8; e += 2) l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e], pb[e + 1]}, ones, l_run, false);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int col = dt * 16 + lr;
    bf16x8 va;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 16 * (e / 4) + 4 * (e % 4) + lg;
      va[e] = static_cast<__bf16>(vb[r * D + 4 * ((col >> 2) ^ vswz<D>(r)) + (col & 3)]);
    }
    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[dt], 0, 0, 0);
  }
}

// LDS rows of k̄ pieces: 4d bytes (k1 then k2, d/8 16-byte chunks each),
// chunk c of row r at c ^ pswz(r): the 16 rows an MFMA operand read takes
// at one chunk index land on 16 different 16-byte bank groups
template <int D>
__device__ __forceinline__ int pswz(int r) { return D == 64 ? (r & 15) : ((r >> 1) & 7); }

// order-preserving image of a float64 logit (-0 folded to +0, so equal
// values give equal keys)
__device__ __forceinline__ unsigned long long order_key(double s) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(s + 0.0);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Exact top-n of one row by a whole workgroup (256 threads).  Float64
// logits: eight lanes per key, each with d/8 channels (sequential fused
// multiply-adds), then a fixed butterfly over the eight, so every key gets
// the same operation order and the loads are whole 128-byte lines.  They are
// kept as order keys in `cache` when m <= cap and recomputed per pass
// otherwise.  Eight 8-bit radix passes find the n-th largest key (a 256-bin
// LDS histogram per pass, each thread adding its runs of equal digits with
// one atomic, the digit found by one wave's scan) and how many keys equal to
// it are taken; an ascending sweep writes the keys above it and the
// lowest-index keys equal to it.  Ends with a barrier, so LDS may be reused.
template <int D>
__device__ __forceinline__ void exact_row(const CSArgs& a, long long slice, int r,
                                          unsigned long long* cache, int cap, double* Qf,
                                          unsigned* Hist, int* Xch) {
  constexpr int E = D / 8;   // channels per lane
  const int m = a.m, n = a.topn;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int sub = lane & 7, kl = lane >> 3;   // channel group, key within the wave's 8
  const double* kslice = a.kbar + (size_t)slice * m * D;
  if (tid < D) Qf[tid] = a.qbar[((size_t)slice * m + r) * D + tid];
  __syncthreads();
  double qreg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qreg[e] = Qf[E * sub + e];
  // order key of key j formed by the 8 lanes kl of this wave (valid in all 8)
  auto coop_key = [&](int j) __attribute__((always_inline)) {
    double s = 0.0;
    if (j < m) {
      const double2* kr = reinterpret_cast<const double2*>(kslice + (size_t)j * D + E * sub);
#pragma unroll
      for (int e = 0; e < E / 2; ++e) {
        const double2 kv = kr[e];
        s = fma(qreg[2 * e], kv.x, s);
        s = fma(qreg[2 * e + 1], kv.y, s);
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    return order_key(s);
  };
  const bool cached = m <= cap;
  if (cached) {
    for (int j0 = 8 * w; j0 < m; j0 += 32) {
      const int j = j0 + kl;
      const unsigned long long x = coop_key(j);
      if (sub == 0 && j < m) cache[j] = x;
    }
  }
  __syncthreads();
  unsigned long long prefix = 0, mask = 0;
  int k = n;   // rank of the wanted key among the keys matching prefix
  for (int shift = 56; shift >= 0; shift -= 8) {
    Hist[tid] = 0u;
    __syncthreads();
    int cur = -1;
    unsigned cnt = 0;
    auto count = [&](unsigned long long x) __attribute__((always_inline)) {
      if ((x & mask) == prefix) {
        const int dg = (int)((x >> shift) & 255);
        if (dg != cur) {
          if (cnt) atomicAdd(&Hist[cur], cnt);
          cur = dg;
          cnt = 0;
        }
        ++cnt;
      }
    };
    if (cached) {
      for (int j = tid; j < m; j += 256) count(cache[j]);
    } else {
      for (int j0 = 8 * w; j0 < m; j0 += 32) {
        const int j = j0 + kl;
        const unsigned long long x = coop_key(j);
        if (sub == 0 && j < m) count(x);
      }
    }
    if (cnt) atomicAdd(&Hist[cur], cnt);
    __syncthreads();
    if (w == 0) {
      // lane l takes bins 255-4l .. 252-4l (descending); exclusive prefix
      // over lanes gives the count of larger digits
      unsigned h[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = Hist[255 - 4 * lane - i];
        tot += h[i];
      }
      unsigned incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const unsigned t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      unsigned acc = incl - tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc < (unsigned)k && (unsigned)k <= acc + h[i]) {
          Xch[0] = 255 - 4 * lane - i;
          Xch[1] = (int)acc;
        }
        acc += h[i];
      }
    }
    __syncthreads();
    prefix |= (unsigned long long)Xch[0] << shift;
    mask |= 0xFFull << shift;
    k -= Xch[1];
    __syncthreads();
  }
  // ascending sweep over keys tid, tid + 256, ...: the block's keys of one
  // step are ordered by thread, so ballots and per-wave counts give each
  // taken key its output slot
  int32_t* out = a.sel + ((size_t)slice * m + r) * n;
  const unsigned long long below = (1ull << lane) - 1;
  int taken = 0, eq_seen = 0;
  for (int base = 0; base < m; base += 256) {
    unsigned long long x = 0;
    if (cached) {
      const int j = base + tid;
      x = j < m ? cache[j] : 0ull;
    } else {
      // the wave's 64 keys base + 64w + o, eight per call: call i forms
      // o = 8i + kl in lanes 8kl .. 8kl+7, and lane 8kl + i keeps it, so lane
      // L holds o = 8(L%8) + L/8; lane t takes its own key o = t from lane
      // 8(t%8) + t/8
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned long long y = coop_key(base + 64 * w + 8 * i + kl);
        if (sub == i) x = y;
      }
      x = __shfl(x, 8 * (lane % 8) + lane / 8);
    }
    const int j = base + tid;
    const bool gt = j < m && x > prefix;
    const bool eq = j < m && x == prefix;
    const unsigned long long eqm = __ballot(eq);
    if (lane == 0) Xch[w] = __popcll(eqm);
    __syncthreads();
    int eq_before = eq_seen + __popcll(eqm & below), eq_all = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      eq_before += u < w ? Xch[u] : 0;
      eq_all += Xch[u];
    }
    const bool take = gt || (eq && eq_before < k);
    const unsigned long long tm = __ballot(take);
    __syncthreads();
    if (lane == 0) Xch[w] = __popcll(tm);
    __syncthreads();
    int pos = taken + __popcll(tm & below), t_all = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pos += u < w ? Xch[u] : 0;
      t_all += Xch[u];
    }
    if (take && pos < n) out[pos] = j;   // exactly n are taken; the bound only guards the buffer
    taken += t_all;
    eq_seen += eq_all;
    __syncthreads();
  }
}

template <int D>
__device__ __forceinline__ void issue_pieces(int c0, uint16_t* pb, float* vb, const char* pbytes,
                                             const char* vbytes, int32x4 rp, int32x4 rv, bool use_rsrc,
                                             int m, int w, int lane) {
  constexpr int PROW = D * 4, VROW = D * 4;   // bytes per LDS row
  constexpr int PLOADS = kCols * PROW / 1024 / 4, VLOADS = kCols * VROW / 1024 / 4;   // 1 KB loads per wave
  static_assert(PLOADS >= 1 && VLOADS >= 1, "chunk split");
  const bool whole = use_rsrc && c0 + kCols <= m;
#pragma unroll
  for (int gg = 0; gg < PLOADS; ++gg) {
    const int g = w + 4 * gg;
    const int byte = 1024 * g + 16 * lane;
    const int r = byte / PROW, pc = (byte % PROW) / 16;
    const int off = r * PROW + 16 * (pc ^ pswz<D>(r));
    char* dst = reinterpret_cast<char*>(pb) + 1024 * g;
    if (whole) dma_buffer(dst, off, rp, c0 * PROW);
    else dma_global(dst, c0 + r < m ? (const void*)(pbytes + (size_t)c0 * PROW + off) : (const void*)&kZero16);
  }
#pragma unroll
  for (int gg = 0; gg < VLOADS; ++gg) {
    const int g = w + 4 * gg;
    const int byte = 1024 * g + 16 * lane;
    const int r = byte / VROW, pc = (byte % VROW) / 16;
    const int off = r * VROW + 16 * (pc ^ vswz<D>(r));
    char* dst = reinterpret_cast<char*>(vb) + 1024 * g;
    if (whole) dma_buffer(dst, off, rv, c0 * VROW);
    else dma_global(dst, c0 + r < m ? (const void*)(vbytes + (size_t)c0 * VROW + off) : (const void*)&kZero16);
  }
}

// Three waves per SIMD (at most 168 VGPRs) run the stage about 15% faster
// than two.  Each lane lists its best eight keys while streaming, and the
// final merges keep all 32 of the row's four lists.  A lane holds about a
// quarter of its row's top n, so eight rarely drops one (and a row whose
// lane did is not certified).  Sixteen per lane, the best 32 kept, ran
// 6% slower at top-16 and 20% slower at top-8.
template <int D>
__global__ __launch_bounds__(256, 3) void compress_select_apx_kernel(CSArgs a) {
  constexpr int K = 8;                   // list entries per lane while streaming
  constexpr int H = D / 32;              // 32-wide halves of d
  constexpr int PE = 2 * D;              // bf16 per row of pieces
  constexpr int kStage = kCols * D * 16;   // bytes: two chunks of pieces and of v̄
  // the staging buffers; after the stream loop the exact fallback keeps a
  // row's logit keys here
  __shared__ __attribute__((aligned(16))) char Stage[kStage];
  uint16_t* const Pb0 = reinterpret_cast<uint16_t*>(Stage);
  uint16_t* const Pb1 = Pb0 + kCols * PE;
  float* const Vb0 = reinterpret_cast<float*>(Pb1 + kCols * PE);
  float* const Vb1 = Vb0 + kCols * D;
  __shared__ float Kmax2[4];
  __shared__ int FailRows[64];
  __shared__ int NFail;
  __shared__ __attribute__((aligned(16))) double Qf[D];
  __shared__ unsigned Hist[256];
  __shared__ int Xch[4];

  long long logical;   // contiguous run of row tiles per XCD
  {
    const long long G = gridDim.x, b = blockIdx.x;
    const long long q8 = G / 8, r8 = G % 8, xcd = b % 8, k = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + k : r8 * (q8 + 1) + (xcd - r8) * q8 + k;
  }
  const int m = a.m;
  const int n = a.topn;
  const int jb = (n + 3) / 4 - 1;   // each lane's entry jb bounds its row's n-th best from below
  const long long slice = logical / a.row_tiles;
  const int tile = (int)(logical % a.row_tiles);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16;   // this lane's row within the wave
  const int lg = lane / 16;   // lane group: keys congruent to lg mod 4
  const int row = tile * 64 + w * 16 + lr;

  const double* qb = a.qbar + (size_t)slice * m * D;
  const double* kslice = a.kbar + (size_t)slice * m * D;
  const char* pbytes = reinterpret_cast<const char*>(a.kpieces + (size_t)slice * m * PE);
  const char* vbytes = reinterpret_cast<const char*>(a.vbar + (size_t)slice * m * D);
  const bool use_rsrc = (long long)m * D * 4 < 0x7fffffffLL;
  const int32x4 rp = slice_rsrc(pbytes, use_rsrc ? m * D * 4 : 0);
  const int32x4 rv = slice_rsrc(vbytes, use_rsrc ? m * D * 4 : 0);
  const float c = (float)a.c_exp2;
  const float lazy = 8.0f / c;

  issue_pieces<D>(0, Pb0, Vb0, pbytes, vbytes, rp, rv, use_rsrc, m, w, lane);

  // q̄ of this lane's row, channels 32h + 8lg + e (the B operand slots of
  // half h), and its pieces
  double qa[D / 4];
#pragma unroll
  for (int hh = 0; hh < H; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) qa[8 * hh + e] = row < m ? qb[(size_t)row * D + 32 * hh + 8 * lg + e] : 0.0;
  bf16x8 q1[H], q2[H];
  double qn2 = 0.0;
#pragma unroll
  for (int hh = 0; hh < H; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = qa[8 * hh + e];
      const __bf16 b1 = static_cast<__bf16>(static_cast<float>(x));
      q1[hh][e] = b1;
      q2[hh][e] = static_cast<__bf16>(static_cast<float>(x - static_cast<double>(static_cast<float>(b1))));
      qn2 = fma(x, x, qn2);
    }
  qn2 += __shfl_xor(qn2, 16);
  qn2 += __shfl_xor(qn2, 32);
  const double qn = sqrt(qn2);

  if (threadIdx.x == 0) NFail = 0;
  // largest |k̄_j|^2 of the slice
  {
    const float* kb2 = a.kbn2 + (size_t)slice * m;
    float mx = 0.f;
    for (int j = threadIdx.x; j < m; j += 256) mx = fmaxf(mx, kb2[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) Kmax2[w] = mx;
  }
  // (the first barrier of the stream loop publishes Kmax2)

  floatx4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  float tv[K];
  int ti[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    tv[j] = -INFINITY;
    ti[j] = 0x7fffffff;
  }
  float rej = -INFINITY;   // largest value this lane's list has let go
  const int pr = 4 * (lr & 3) + (lr >> 2);   // A row lr of a 16-key tile holds key pr
  float eps = 0.f;

  auto chunk = [&](int c0, const uint16_t* pb, const float* vb) __attribute__((always_inline)) {
    floatx4 acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * ct + pr;
      const uint16_t* prow = pb + r * PE;
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        const int c1 = 4 * hh + lg, c2 = D / 8 + 4 * hh + lg;   // logical 16-byte chunks of k1, k2
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(prow + 8 * (c1 ^ pswz<D>(r)));
        const bf16x8 k2 = *reinterpret_cast<const bf16x8*>(prow + 8 * (c2 ^ pswz<D>(r)));
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, q1[hh], acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k2, q1[hh], acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, q2[hh], acc[ct], 0, 0, 0);
      }
    }
    if (c0 + kCols > m) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 16 * ct + 4 * i + lg >= m) acc[ct][i] = -INFINITY;
    }
    chunk_softmax_pv_f<D>(acc, vb, c, lazy, m_run, l_run, oacc, lr, lg);
    // keys within 4ε below a lower bound of the row's n-th best are kept
    float bound = tv[0];
#pragma unroll
    for (int j = 1; j < K && j < 4; ++j)
      if (jb == j) bound = tv[j];
    bound = fminf(bound, __shfl_xor(bound, 16));
    bound = fminf(bound, __shfl_xor(bound, 32));
    const float low = bound - 4.0f * eps;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc[ct][i];
        float dropped = x;
        if (__ballot(x > tv[K - 1] && x >= low)) {
          dropped = x > tv[K - 1] ? tv[K - 1] : x;
          list_insert_f<K>(tv, ti, x, c0 + 16 * ct + 4 * i + lg);
        }
        rej = fmaxf(rej, dropped);
      }
  };

  // stream: wait for chunk c, then (every wave being past chunk c-1) load
  // chunk c+1 into the other buffers while chunk c is computed
  for (int c0 = 0; c0 < m; c0 += kCols) {
    const int par = (c0 / kCols) & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (c0 == 0) {
      const float k2 = fmaxf(fmaxf(Kmax2[0], Kmax2[1]), fmaxf(Kmax2[2], Kmax2[3]));
      eps = (float)(kApxEps * qn * sqrt((double)k2)) * 1.0001f;
    }
    if (c0 + kCols < m)
      issue_pieces<D>(c0 + kCols, par ? Pb0 : Pb1, par ? Vb0 : Vb1, pbytes, vbytes, rp, rv, use_rsrc, m, w, lane);
    chunk(c0, par ? Pb1 : Pb0, par ? Vb1 : Vb0);
  }

  store_ocg<D>(a.o_cg + ((size_t)slice * m + row) * D, oacc, l_run, lg, row < m);

  // the row's 4K keys: merge the lane groups pairwise, without loss
  constexpr int L = 2 * K;
  float lv[L];
  int li[L];
  {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      lv[j] = tv[j];
      li[j] = ti[j];
      lv[L - 1 - j] = __shfl_xor(tv[j], 16);   // partner's list reversed: a bitonic sequence
      li[L - 1 - j] = __shfl_xor(ti[j], 16);
    }
    bitonic_merge_f<L>(lv, li);
  }
  rej = fmaxf(rej, __shfl_xor(rej, 16));
  // the row's best 32 (kept in every lane of the row)
  constexpr int LF = 32;
  float fv[LF];
  int fi[LF];
  {
    float pv[L];
    int pi[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      pv[j] = __shfl_xor(lv[j], 32);
      pi[j] = __shfl_xor(li[j], 32);
    }
    static_assert(2 * L == LF, "the two halves fill the final list");
    // the partner's list reversed makes one bitonic sequence, merged without loss
#pragma unroll
    for (int j = 0; j < L; ++j) {
      fv[j] = lv[j];
      fi[j] = li[j];
      fv[LF - 1 - j] = pv[j];
      fi[LF - 1 - j] = pi[j];
    }
    bitonic_merge_f<LF>(fv, fi);
  }
  rej = fmaxf(rej, __shfl_xor(rej, 32));

  // certification and the band around the n-th value
  float vn = fv[0];
#pragma unroll
  for (int j = 1; j < 16; ++j)
    if (j == n - 1) vn = fv[j];
  const float band_lo = vn - 2.0f * eps, band_hi = vn + 2.0f * eps;
  int above = 0, inband = 0;
#pragma unroll
  for (int j = 0; j < LF; ++j) {
    above += fv[j] > band_hi ? 1 : 0;
    inband += (fv[j] >= band_lo && fv[j] <= band_hi) ? 1 : 0;
  }
  static_assert(16 + kBandMax <= 32, "result slots");
  bool ok = rej < band_lo && inband <= kBandMax;
  // the wave's largest band among certified rows: band work stops there
  int bmax = ok ? inband : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bmax = max(bmax, __shfl_xor(bmax, o));
  // band entries (positions above .. above+inband-1 of the sorted list)
  int bidx[kBandMax];
#pragma unroll
  for (int t = 0; t < kBandMax; ++t) {
    int v = 0x7fffffff;
    if (t < bmax) {
#pragma unroll
      for (int j = 0; j < LF; ++j)
        if (j == above + t) v = fi[j];
    }
    bidx[t] = t < inband ? v : 0x7fffffff;
  }
  // exact rescoring: each lane forms its channels' share (32h + 8lg + e)
  // with the same fused multiply-adds in the same order for every key, then
  // the row's four lanes add their shares in a fixed pairing
  double ex[kBandMax];
#pragma unroll
  for (int t = 0; t < kBandMax; ++t) {
    ex[t] = -INFINITY;
    if (t < bmax) {
      const int kj = (t < inband && bidx[t] < m) ? bidx[t] : 0;
      const double* kr = kslice + (size_t)kj * D + 8 * lg;
      double part = 0.0;
#pragma unroll
      for (int hh = 0; hh < H; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fma(qa[8 * hh + e], kr[32 * hh + e], part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      ex[t] = part;
    }
  }
  const int need = n - above;
  int ix[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) ix[j] = j < above ? fi[j] : 0x7fffffff;
#pragma unroll
  for (int t = 0; t < kBandMax; ++t) {
    int rank = 0;
    if (t < bmax) {
#pragma unroll
      for (int u = 0; u < kBandMax; ++u)
        if (u < bmax && u < inband && u != t && (ex[u] > ex[t] || (ex[u] == ex[t] && bidx[u] < bidx[t]))) ++rank;
    }
    ix[16 + t] = (t < inband && rank < need) ? bidx[t] : 0x7fffffff;
  }
#pragma unroll
  for (int t = 16 + kBandMax; t < 32; ++t) ix[t] = 0x7fffffff;
  // ascending block order (bitonic sort of 32)
#pragma unroll
  for (int k = 2; k <= 32; k <<= 1)
#pragma unroll
    for (int sd = k / 2; sd >= 1; sd >>= 1)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if ((j & sd) == 0) {
          const bool up = (j & k) == 0;
          const int lo = min(ix[j], ix[j + sd]), hi = max(ix[j], ix[j + sd]);
          ix[j] = up ? lo : hi;
          ix[j + sd] = up ? hi : lo;
        }
  if (row < m && ok) {
    int32_t* dst = a.sel + ((size_t)slice * m + row) * n;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j / 4 == lg && j < n) dst[j] = ix[j];
  }

  // rows left uncertified: exact, one at a time, by the whole workgroup
  const bool fail = !ok && lg == 0 && row < m;
  const unsigned long long fm = __ballot(fail);
  if (fm) {
    int base = 0;
    if (lane == 0) base = atomicAdd(&NFail, __popcll(fm));
    base = __shfl(base, 0);
    if (fail) FailRows[base + __popcll(fm & ((1ull << lane) - 1))] = row;
  }
  __syncthreads();   // every wave is past the stream loop: Stage is free
  const int nfail = NFail;
  if (nfail > kExactRows) {
    // many rows (crowded logits): the float64 list kernel redoes the tile
    if ((int)threadIdx.x < nfail) a.sel[((size_t)slice * m + FailRows[threadIdx.x]) * n] = -1;
    return;
  }
  for (int f = 0; f < nfail; ++f)
    exact_row<D>(a, slice, FailRows[f], reinterpret_cast<unsigned long long*>(Stage), kStage / 8, Qf, Hist, Xch);
}

// ---------------------------------------------------------------------------
// Buffered kernel: exact for any n <= 64, one workgroup per row tile.

template <int D>
__global__ __launch_bounds__(256) void compress_select_buffered_kernel(CSArgs a) {
  __shared__ __attribute__((aligned(16))) double Kb0[kCols * D];
  __shared__ __attribute__((aligned(16))) float Vb0[kCols * D];
  __shared__ __attribute__((aligned(16))) double Kb1[kCols * D];
  __shared__ __attribute__((aligned(16))) float Vb1[kCols * D];
  // candidate buffers, rows padded by 16 entries so that neighbouring rows
  // start in different LDS bank halves (a row is 1 KB unpadded)
  __shared__ double BufV[64][kCap + 16];
  __shared__ int BufI[64][kCap + 16];
  __shared__ int Cnt[64];
  __shared__ double ThrV[64];
  __shared__ int ThrI[64];

  const int m = a.m;
  const int n = a.topn;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // scalar: uniform branches
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16;   // this lane's row within the wave
  const int lg = lane / 16;   // lane group 0..3
  const int brow = w * 16 + lr;   // this lane's row in the workgroup buffers
  const long long slice = (long long)blockIdx.x / a.row_tiles;
  const int tile = (int)(blockIdx.x % a.row_tiles);

  const double* qb = a.qbar + (size_t)slice * m * D;
  const char* kbytes = reinterpret_cast<const char*>(a.kbar + (size_t)slice * m * D);
  const char* vbytes = reinterpret_cast<const char*>(a.vbar + (size_t)slice * m * D);
  const bool use_rsrc = (long long)m * D * 8 < 0x7fffffffLL;   // 32-bit buffer offsets
  const int32x4 rk = slice_rsrc(kbytes, use_rsrc ? m * D * 8 : 0);
  const int32x4 rv = slice_rsrc(vbytes, use_rsrc ? m * D * 4 : 0);
  const double lazy = 8.0 / a.c_exp2;   // 2^8 in weight, in units of raw dot products

  {
    const int rw = tile * 64 + w * 16;
    if (threadIdx.x < 64) {
      Cnt[threadIdx.x] = 0;
      ThrV[threadIdx.x] = -INFINITY;
      ThrI[threadIdx.x] = 0x7fffffff;
    }

    double qa[D / 4];
    {
      const int row = rw + lr;
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) qa[ks] = row < m ? qb[(size_t)row * D + 4 * ks + lg] : 0.0;
    }

    floatx4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    double m_run = -INFINITY;
    float l_run = 0.f;
    double thr_v = -INFINITY;   // current n-th best key of row lr
    int thr_i = 0x7fffffff;

    // Sort the buffers of rows R0 .. R0+3 (16 lanes each) and keep each row's
    // best n; with final set, write them out in ascending block order instead.
    auto compact4 = [&](int R0, bool final) __attribute__((always_inline)) {
      const int R = R0 + lg, l = lr;
      const int c = Cnt[R];
      double v[8];
      int ix[8];
      // unsorted input, so any placement will do: read buffer entry 16*e + l
      // into slot e of lane l (16 lanes read 16 consecutive entries)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = 16 * e + l;
        v[e] = pos < c ? BufV[R][pos] : -INFINITY;
        ix[e] = pos < c ? BufI[R][pos] : 0x7fffffff;
      }
      sort_rows4(v, ix, l);   // now position 8*l + e holds the (8*l+e)-th best
      if (!final) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = 8 * l + e;
          if (pos < n) {
            BufV[R][pos] = v[e];
            BufI[R][pos] = ix[e];
          }
          if (pos == n - 1) {
            ThrV[R] = v[e];
            ThrI[R] = ix[e];
            Cnt[R] = n;
          }
        }
      } else {
        // the best n, by block index: rank among the kept n through LDS
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * l + e < n) BufI[R][8 * l + e] = ix[e];
        wave_sync_lds();
        const int row = tile * 64 + R;
        if (row < m) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pos = 8 * l + e;
            if (pos < n) {
              int rank = 0;
              for (int j = 0; j < n; ++j) rank += BufI[R][j] < ix[e] ? 1 : 0;
              a.sel[((size_t)slice * m + row) * n + rank] = ix[e];
            }
          }
        }
      }
    };

    auto chunk = [&](int c0, const double* kb, const float* vb) __attribute__((always_inline)) {
      doublex4 acc[2];
      chunk_logits<D>(acc, kb, qa, c0, m, lr, lg);
      chunk_softmax_pv<D>(acc, vb, a.c_exp2, lazy, m_run, l_run, oacc, lr, lg);

      // selection: append the logits that beat the row's current n-th key.
      // The four lanes of a row (lanes lr, lr+16, lr+32, lr+48) take
      // consecutive slots by a prefix count, so no atomics are needed.
      unsigned cm = 0;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = c0 + 16 * ct + 4 * i + lg;
          if (col < m && beats(acc[ct][i], col, thr_v, thr_i)) cm |= 1u << (4 * ct + i);
        }
      if (__ballot(cm != 0)) {
        const int mine = __popc(cm);
        const int up16 = __shfl_xor(mine, 16);
        const int up32 = __shfl_xor(mine, 32);
        const int up48 = __shfl_xor(up16, 32);
        // counts of lane groups 0..3 of this row, in group order
        const int c_g0 = lg == 0 ? mine : (lg == 1 ? up16 : (lg == 2 ? up32 : up48));
        const int c_g1 = lg == 1 ? mine : (lg == 0 ? up16 : (lg == 3 ? up32 : up48));
        const int c_g2 = lg == 2 ? mine : (lg == 3 ? up16 : (lg == 0 ? up32 : up48));
        const int c_g3 = lg == 3 ? mine : (lg == 2 ? up16 : (lg == 1 ? up32 : up48));
        int pos = Cnt[brow] + (lg > 0 ? c_g0 : 0) + (lg > 1 ? c_g1 : 0) + (lg > 2 ? c_g2 : 0);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (cm & (1u << (4 * ct + i))) {
              BufV[brow][pos] = acc[ct][i];
              BufI[brow][pos] = c0 + 16 * ct + 4 * i + lg;
              ++pos;
            }
        __builtin_amdgcn_wave_barrier();
        if (lg == 0) Cnt[brow] += c_g0 + c_g1 + c_g2 + c_g3;
      }
      wave_sync_lds();

      // compact rows whose buffer passed kCap - kCols entries (the next chunk
      // adds at most kCols): one read of the wave's 16 counts, a ballot, then
      // each group of four rows holding such a row is sorted together
      const unsigned long long full = __ballot(lane < 16 && Cnt[w * 16 + (lane & 15)] > kCap - kCols);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((full >> (4 * q)) & 0xF) compact4(w * 16 + 4 * q, false);
      wave_sync_lds();
      thr_v = ThrV[brow];
      thr_i = ThrI[brow];
    };

    // double-buffered stream over the key blocks (the counters above are
    // published by the first barrier)
    issue_chunk<D>(0, Kb0, Vb0, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    for (int c0 = 0; c0 < m; c0 += 2 * kCols) {
      if (c0 + kCols < m) issue_chunk<D>(c0 + kCols, Kb1, Vb1, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
      chunk(c0, Kb0, Vb0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (c0 + kCols >= m) break;
      if (c0 + 2 * kCols < m) issue_chunk<D>(c0 + 2 * kCols, Kb0, Vb0, kbytes, vbytes, rk, rv, use_rsrc, m, w, lane);
      chunk(c0 + kCols, Kb1, Vb1);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    }

    store_ocg<D>(a.o_cg + ((size_t)slice * m + rw + lr) * D, oacc, l_run, lg, rw + lr < m);

    // final top-n of every row, written in ascending block order
    wave_sync_lds();
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (rw + 4 * q < m) compact4(w * 16 + 4 * q, true);
  }
}

// ---------------------------------------------------------------------------
// Any top-n (used for n > 64): one wave per row, exact radix selection.
//
// The lane-list and buffered kernels above keep at most 64 candidates per
// row.  This kernel selects any n <= m.  A wave owns one query-block row and
// streams the slice's key blocks, lane l taking keys l, l+64, ...; every
// pass recomputes the row's float64 logits (the same fused multiply-adds in
// the same order each time, so every pass sees identical values):
//   1. the row maximum;
//   2. ā_ij = 2^((s_ij - max)·log2(e)/sqrt(d)) in float32 and
//      o_CG_i = sum_j ā_ij v̄_j / sum_j ā_ij, lane l accumulating dimension l
//      while each key's weight is broadcast from the lane that formed it;
//   3. eight 8-bit radix passes over an order-preserving 64-bit image of the
//      logits find the n-th largest value V exactly (a 256-bin LDS histogram
//      per wave and pass) and how many of the keys equal to V belong to the
//      top n;
//   4. an ascending sweep writes every j with s_ij > V, and the lowest-index
//      keys with s_ij = V, in ascending order (ballot prefix counts).
// The logits are float64 dot products of the exact block means, ranked raw
// (dividing by sqrt(d) is monotone), so the selection equals a float64
// evaluation up to the summation order of the products; -0 is folded to +0
// so that equal logits compare equal.  Cost: about 11 recomputations of the
// row's m logits; this path serves shapes the fast kernels do not cover.
__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void compress_select_generic_kernel(CSArgs a, long long rows) {
  __shared__ __attribute__((aligned(16))) double Qs[4][D];
  __shared__ unsigned Hist[4][256];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const long long grow = (long long)blockIdx.x * 4 + w;   // slice * m + row
  if (grow >= rows) return;   // whole waves only; no workgroup barrier below
  const int m = a.m, n = a.topn;
  const long long slice = grow / m;
  const double2* kb = reinterpret_cast<const double2*>(a.kbar + (size_t)slice * m * D);
  const float* vb = a.vbar + (size_t)slice * m * D;
  for (int d = lane; d < D; d += kWave) Qs[w][d] = a.qbar[(size_t)grow * D + d];
  wave_sync_lds();
  const double2* qs = reinterpret_cast<const double2*>(Qs[w]);
  auto dot = [&](int j) __attribute__((always_inline)) -> double {
    const double2* kr = kb + (size_t)j * (D / 2);
    double s = 0.0;
#pragma unroll 8
    for (int e = 0; e < D / 2; ++e) {
      const double2 kv = kr[e], qv = qs[e];
      s = fma(qv.x, kv.x, s);
      s = fma(qv.y, kv.y, s);
    }
    return s;
  };

  // 1. row maximum
  double mx = -INFINITY;
  for (int j = lane; j < m; j += kWave) mx = fmax(mx, dot(j));
  mx = wave_max_f64(mx);

  // 2. softmax weights and o_CG
  float o = 0.f, lsum = 0.f;
  for (int base = 0; base < m; base += kWave) {
    const int j = base + lane;
    const float p = j < m ? __builtin_amdgcn_exp2f((float)((dot(j) - mx) * a.c_exp2)) : 0.f;
    lsum += p;
    const int cnt = min(kWave, m - base);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj);
      if (lane < D) o = fmaf(pj, vb[(size_t)(base + jj) * D + lane], o);
    }
  }
  lsum = wave_sum_f32(lsum);
  if (lane < D) a.o_cg[(size_t)grow * D + lane] = o / lsum;

  // 3. radix selection of the n-th largest key
  unsigned long long prefix = 0, mask = 0;
  int k = n;   // rank of the wanted key among the keys matching `prefix`
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int e = lane; e < 256; e += kWave) Hist[w][e] = 0u;
    wave_sync_lds();
    for (int j = lane; j < m; j += kWave) {
      const unsigned long long kk = order_key(dot(j));
      if ((kk & mask) == prefix) atomicAdd(&Hist[w][(kk >> shift) & 255], 1u);
    }
    wave_sync_lds();
    int dd = 0, above = 0;
    if (lane == 0) {
      int acc = 0;
      for (dd = 255; dd > 0; --dd) {
        const int h = (int)Hist[w][dd];
        if (acc + h >= k) break;
        acc += h;
      }
      above = acc;
    }
    dd = __shfl(dd, 0);
    above = __shfl(above, 0);
    prefix |= (unsigned long long)dd << shift;
    mask |= 0xFFull << shift;
    k -= above;
    wave_sync_lds();
  }

  // 4. ascending sweep: keys above the n-th value, then the k lowest-index
  // keys equal to it
  int32_t* out = a.sel + (size_t)grow * n;
  int taken = 0, eq_seen = 0;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < m; base += kWave) {
    const int j = base + lane;
    const unsigned long long kk = j < m ? order_key(dot(j)) : 0ull;
    const bool gt = j < m && kk > prefix;
    const bool eq = j < m && kk == prefix;
    const unsigned long long eqm = __ballot(eq);
    const bool take = gt || (eq && eq_seen + __popcll(eqm & below) < k);
    const unsigned long long tm = __ballot(take);
    const int pos = taken + __popcll(tm & below);
    if (take && pos < n) out[pos] = j;   // exactly n are taken; the bound only guards the buffer
    taken += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
}

}  // namespace

hipError_t launch_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                  float* o_cg, int32_t* sel, long long slices, int m, int head_dim,
                                  int topn, hipStream_t stream, const uint16_t* kpieces,
                                  const float* kbn2) {
  CSArgs a;
  a.kpieces = kpieces;
  a.kbn2 = kbn2;
  a.qbar = qbar;
  a.kbar = kbar;
  a.vbar = vbar;
  a.o_cg = o_cg;
  a.sel = sel;
  a.m = m;
  a.topn = topn;
  a.row_tiles = (m + 63) / 64;
  a.c_exp2 = 1.4426950408889634 / sqrt((double)head_dim);
  a.redo = 0;
  const dim3 grid((unsigned)(slices * a.row_tiles));
  if (topn <= 16 && kpieces && kbn2) {   // approximate logits, certified; crowded tiles redone in float64
    if (head_dim == 64) hipLaunchKernelGGL(compress_select_apx_kernel<64>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(compress_select_apx_kernel<32>, grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.redo = 1;
  }
  if (topn > 64) {   // beyond the candidate capacity of the fast kernels
    const long long rows = slices * (long long)m;
    const dim3 ggrid((unsigned)((rows + 3) / 4));
    if (head_dim == 64)
      hipLaunchKernelGGL(compress_select_generic_kernel<64>, ggrid, dim3(256), 0, stream, a, rows);
    else
      hipLaunchKernelGGL(compress_select_generic_kernel<32>, ggrid, dim3(256), 0, stream, a, rows);
    return hipGetLastError();
  }
  if (head_dim == 64) {
    if (topn <= 8) hipLaunchKernelGGL((compress_select_list_kernel<64, 8>), grid, dim3(256), 0, stream, a);
    else if (topn <= 16) hipLaunchKernelGGL((compress_select_list_kernel<64, 16>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(compress_select_buffered_kernel<64>, grid, dim3(256), 0, stream, a);
  } else {
    if (topn <= 8) hipLaunchKernelGGL((compress_select_list_kernel<32, 8>), grid, dim3(256), 0, stream, a);
    else if (topn <= 16) hipLaunchKernelGGL((compress_select_list_kernel<32, 16>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(compress_select_buffered_kernel<32>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mosaic
