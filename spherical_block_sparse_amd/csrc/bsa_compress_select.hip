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
//   * buffered kernel (16 < n <= 64): each row keeps
//     its current n-th best key; logits that beat it are appended to an LDS
//     candidate buffer at prefix-count slots, and a buffer that could
//     overflow is compacted to its best n by a 128-entry bitonic network over
//     four rows at once (register and DPP / swizzle exchanges).
// Roofline: float64 matrix work 2*m^2*d per slice for the logits plus bf16
// matrix work 2*m^2*d for ā·v̄; HBM traffic is only the pooled tensors, o_CG
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
  const dim3 grid((unsigned)(slices * a.row_tiles));
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
