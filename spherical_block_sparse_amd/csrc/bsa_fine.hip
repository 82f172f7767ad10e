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
//   * a workgroup owns T = 32*WAVES consecutive queries of one slice (T = 64
//     for blocks of 64 tokens, 128 when a block holds >= 128 tokens so that
//     more queries share one gathered key set); each wave owns 32 queries as
//     two 16-query sub-tiles whose MFMAs share every K / V operand read.
//   * keys stream into LDS 64 at a time with gfx950 direct loads to LDS
//     (lane l of a wave's 16-byte load writes bytes 16*l..16*l+15 of a 1 KB
//     span): buffer loads with fixed per-lane offsets and the chunk start as
//     a scalar offset for runs of 64 consecutive tokens, global loads for
//     gathered or partial chunks.  K and V are row-major [key][d] with the
//     16-byte chunks of each row XOR-swizzled; two K/V buffer pairs in one
//     LDS array, so the loads of chunk c+1 are in flight while chunk c is
//     computed, one barrier per chunk, no staging registers.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 keys x 16 queries per
//     tile); in that layout each lane owns 16 scores of one query, so the
//     online softmax needs two cross-lane steps per chunk and the
//     bf16-rounded weights are already the B operand of O^T += V^T P^T.
//   * the V^T operand is read with the gfx950 transposing LDS load
//     ds_read_b64_tr_b16: within each group of 16 lanes, output lane i
//     receives element i%4 of the 8-byte rows addressed by source lanes
//     4j + i/4 (j = 0..3), so source lane r of group g points at key
//     32*jj + 16*h + 4*g + r/4, column 16*dt + 4*(r%4).
//   * softmax in base 2 with log2(e)/sqrt(d) folded into the scores; the
//     running reference max only moves when a score exceeds it by more than
//     2^8 (weights stay <= 256), so O is rescaled on few chunks.  Given the
//     pool's largest key norm per key block, a query's scores over a
//     branch's blocks are bounded by c*|q|*max|k|; when those bounds are small
//     enough for every query of a wave, the bounds serve as fixed
//     references and the running maximum is skipped altogether.  The
//     selected branch's max|k| per query block can come precomputed
//     (sel_bound_kernel, launched by the caller between the selection and
//     this kernel); without it the prologue gathers it.  The
//     denominator is the same MFMA with an all-ones A operand (sum of the
//     rounded weights, so each output is an exact convex combination of the
//     weights actually applied).
//   * selected branch: virtual key v of a group -> token sel[v/block]*block +
//     v%block; for blocks smaller than T the tile's T/block query blocks are
//     taken in turn by the sub-tiles they contain.
//   * local branch: the union of the tile's windows is streamed; chunks
//     inside every window of a sub-tile run unmasked, chunks outside it are
//     skipped, the rest are masked per score.
//   * workgroup ids are remapped so each XCD (dispatched round-robin) gets a
//     contiguous run of tiles: neighbouring tiles share window keys and
//     largely the same selected blocks, and they now share an L2.
//   * epilogue: out = g0·o_CG[t/block] + g1·o_FG + g2·o_L, float32.  The
//     SAVE instantiation (training forward) also stores o_FG, o_L (float32)
//     and their log2-sum-exp, which the backward reads instead of
//     recomputing both branches; the MERGED instantiation (encoder layer)
//     writes out in bf16 with the heads side by side, [b][N][H][D], the
//     layout the output projection reads.
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
  const float* knorm; // largest key norm of each key block [S][m], or null
  const float* selmax;// per query block, the largest of knorm over its selected blocks [S][m], or null
  float* out;
  float* save_o;      // [S][N][2][D] o_FG, o_L (normalised), SAVE only
  float* save_lse;    // [S][N][2] their log2-sum-exp (log2 units of S*log2(e)/sqrt(d)), SAVE only
  uint16_t* out_merged;   // bf16 [b][N][H][D] in place of out, MERGED only
  int heads;
  int n_tok;
  int block;
  int topn;
  int window;
  int m;
  int tiles;          // query tiles per slice
  long long groups;   // total workgroups
  float scale_log2;   // log2(e) / sqrt(d)
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;


constexpr float kLazy = 8.0f;
// entries of the tiled kernel's LDS table of selection rows (T/block rows of
// topn, one row when block >= T); larger selections take the generic kernel
constexpr int kSelTable = 256;
// Largest score bound M (log2 units) for which the running maximum is
// skipped.  The best key's weight is then at least 2^-2M = 2^-96: it, the
// denominator and its products with v elements above 2^-30 stay normal
// float32 and bf16 numbers, 30 binades above the smallest.
constexpr float kBoundMax = 48.0f;


// transposing 8-byte LDS read (ds_read_b64_tr_b16)
__device__ __forceinline__ shortx4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

template <int D>
struct Tile {
  static constexpr int KK = D / 32;   // bf16 k-steps over d for S = K Q^T
  static constexpr int DT = D / 16;   // 16-row tiles of O^T over d
};

// XOR swizzle of the 16-byte chunks of an LDS row (rows are D*2 bytes, no
// padding, so a 1 KB direct load fills whole rows).  For D = 64 it keeps both
// the 16-row K operand reads and the transposing V reads free of bank
// conflicts; for D = 32 the K reads.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return 2 * ((row >> 1) & 3) + ((row >> 3) & 1);
  else return (row >> 2) & 3;
}

template <int D>
struct Branch {               // online-softmax state of one 16-query sub-tile
  floatx4 o[Tile<D>::DT];     // O^T: lane holds d = 16*dt + 4*lg + i of query lr
  floatx4 l;                  // denominator (all four entries equal)
  float m;                    // reference max, log2 units
};

template <int D>
__device__ __forceinline__ void branch_init(Branch<D>& b) {
#pragma unroll
  for (int dt = 0; dt < Tile<D>::DT; ++dt) b.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  b.l = floatx4{0.f, 0.f, 0.f, 0.f};
  b.m = -INFINITY;
}

// P·V for both sub-tiles (and the denominators, as an all-ones A operand);
// act[s] false skips sub-tile s.
template <int D, bool ALL>
__device__ __forceinline__ void pv_chunk(const uint16_t* Vs, const bf16x8 (&pb)[2][2], Branch<D> (&br)[2],
                                         const bool (&act)[2]) {
  constexpr int DT = Tile<D>::DT;
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, lg = lane / 16;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (ALL || act[s]) br[s].l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[s][j], br[s].l, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      // A operand V^T[d = 16*dt + lr][k-slots 8*lg + e]; slot e holds key
      // 32*j + 16*(e/4) + 4*lg + e%4, the order of the scores in pb[s][j]
      // (swz(row + 16) == swz(row), so the second half is 16 rows further)
      const int row = 32 * j + 4 * lg + (lr >> 2);
      const int col = dt * 16 + 4 * (lr & 3);
      const uint16_t* src = Vs + row * D + 8 * ((col >> 3) ^ swz<D>(row)) + (col & 7);
      const shortx4 lo = lds_read_tr16(src);
      const shortx4 hi = lds_read_tr16(src + 16 * D);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (ALL || act[s]) br[s].o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[s][j], br[s].o[dt], 0, 0, 0);
    }
  }
}

// S^T tiles of both sub-tiles: acc[s][kt][i] = q_(lr) . k_(16*kt + 4*lg + i)
template <int D, bool ALL>
__device__ __forceinline__ void qk_chunk(const uint16_t* Ks, const bf16x8 (&qf)[2][Tile<D>::KK],
                                         floatx4 (&acc)[2][4], const bool (&act)[2]) {
  constexpr int KK = Tile<D>::KK;
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, lg = lane / 16;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[s][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int row = kt * 16 + lr;
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + row * D + 8 * ((4 * kk + lg) ^ swz<D>(row)));
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (ALL || act[s]) acc[s][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s][kk], acc[s][kt], 0, 0, 0);
    }
}

// Online-softmax update of the sub-tiles in `act` from raw scores acc (the
// scale c = log2(e)/sqrt(d) is applied inside the exp2 argument).  The
// reference max moves only when a score exceeds it by more than 2^8 after
// scaling.  Each lane checks its own 16 scores of a query against the
// query's reference and the wave votes, so the common case needs no
// exchange between lanes; only when some score grew does the wave form the
// queries' maxima across their four lanes and rescale (a scalar branch; any
// query may move its reference: alpha <= 1 is always exact).  A bounded
// wave's references are fixed upper bounds of its scores, so it skips all
// of this.
template <int D, bool ALL, bool BOUNDED>
__device__ __forceinline__ void softmax_chunk(floatx4 (&acc)[2][4], Branch<D> (&br)[2], bf16x8 (&pb)[2][2],
                                              const bool (&act)[2], float c, float lazy_raw) {
  constexpr int DT = Tile<D>::DT;
  if constexpr (!BOUNDED) {   // bounded references never move
    float mx[2];   // this lane's maximum of each sub-tile's scores
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float a = fmaxf(acc[s][0][0], acc[s][0][1]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = (kt == 0 ? 2 : 0); i < 4; i += 2) a = fmaxf(a, fmaxf(acc[s][kt][i], acc[s][kt][i + 1]));
      mx[s] = a;
    }
    const bool grow = (ALL || act[0]) && mx[0] > br[0].m + lazy_raw;
    const bool grow1 = (ALL || act[1]) && mx[1] > br[1].m + lazy_raw;
    if (__ballot(grow || grow1)) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (!(ALL || act[s])) continue;
        float row = fmaxf(mx[s], __shfl_xor(mx[s], 16));
        row = fmaxf(row, __shfl_xor(row, 32));
        const float mnew = fmaxf(br[s].m, row);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((br[s].m - mnew) * c);
        br[s].m = mnew;
        br[s].l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) br[s].o[dt] *= alpha;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (!(ALL || act[s])) continue;
    const float nmc = br[s].m == -INFINITY ? 0.f : -br[s].m * c;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pb[s][kt >> 1][4 * (kt & 1) + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(acc[s][kt][i], c, nmc)));
  }
}

// One staged 64-key chunk in which both sub-tiles take part (the common
// case).  With MASK, chunk key kappa is valid for this lane's query of
// sub-tile s iff lo[s] <= kappa < lo[s] + span[s] (span >= 0); otherwise
// every key is valid.
template <int D, bool MASK, bool BOUNDED>
__device__ __forceinline__ void attend_full(const uint16_t* Ks, const uint16_t* Vs,
                                            const bf16x8 (&qf)[2][Tile<D>::KK], Branch<D> (&br)[2],
                                            float c, float lazy_raw, const int (&lo)[2], const int (&span)[2]) {
  const bool act[2] = {true, true};
  floatx4 acc[2][4];
  bf16x8 pb[2][2];
  qk_chunk<D, true>(Ks, qf, acc, act);
  if constexpr (MASK) {
    const int lg = (threadIdx.x % kWave) / 16;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((unsigned)(16 * kt + 4 * lg + i - lo[s]) >= (unsigned)span[s]) acc[s][kt][i] = -INFINITY;
  }
  softmax_chunk<D, true, BOUNDED>(acc, br, pb, act, c, lazy_raw);
  pv_chunk<D, true>(Vs, pb, br, act);
}

// One staged 64-key chunk in general form: act[s] says whether sub-tile s
// takes part, msk[s] whether its scores need valid(s, kappa).
template <int D, bool BOUNDED, typename V>
__device__ __forceinline__ void attend_chunk(const uint16_t* Ks, const uint16_t* Vs,
                                             const bf16x8 (&qf)[2][Tile<D>::KK], Branch<D> (&br)[2],
                                             const bool (&act)[2], const bool (&msk)[2], float c,
                                             float lazy_raw, V valid) {
  if (!act[0] && !act[1]) return;
  const int lg = (threadIdx.x % kWave) / 16;
  floatx4 acc[2][4];
  bf16x8 pb[2][2];
  qk_chunk<D, false>(Ks, qf, acc, act);
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (act[s] && msk[s]) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!valid(s, 16 * kt + 4 * lg + i)) acc[s][kt][i] = -INFINITY;
    }
  softmax_chunk<D, false, BOUNDED>(acc, br, pb, act, c, lazy_raw);
  pv_chunk<D, false>(Vs, pb, br, act);
}

constexpr int kNoRange[2] = {0, 0};   // key range argument of unmasked chunks

// 16 zero bytes: the DMA source of key slots that hold no token (masked keys
// then read exact zeros, as a zero-filled chunk would hold)
__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};


// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkm and exp counters not waited on)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

enum FineMode { kPlain = 0, kSave = 1, kMerged = 2 };

template <int D, int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void fine_kernel(FineArgs a) {
  constexpr int KK = Tile<D>::KK, DT = Tile<D>::DT;
  constexpr int T = 32 * WAVES;           // queries per workgroup
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int RPG = 64 / CPR;           // key rows per 1 KB load (one wave instruction)
  constexpr int GPC = 64 / RPG;           // 1 KB loads per tensor per 64-key chunk
  static_assert(GPC % WAVES == 0, "loads split evenly over the waves");
  // the two K/V buffer pairs in one array, 64*D bf16 each: K0, V0, K1, V1
  // (the loads address them from one scalar base plus immediate offsets)
  __shared__ __attribute__((aligned(16))) uint16_t KVb[4 * 64 * D];
  uint16_t* const Kb0 = KVb;
  uint16_t* const Vb0 = KVb + 64 * D;
  uint16_t* const Kb1 = KVb + 2 * 64 * D;
  uint16_t* const Vb1 = KVb + 3 * 64 * D;
  __shared__ int SelT[kSelTable];   // selection rows of the tile's query blocks

  // contiguous run of tiles per XCD (workgroups are dispatched round-robin)
  long long logical;
  {
    const long long G = a.groups, b = blockIdx.x;
    const long long q8 = G / 8, r8 = G % 8, xcd = b % 8, k = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + k : r8 * (q8 + 1) + (xcd - r8) * q8 + k;
  }
  const int N = a.n_tok, B = a.block, n = a.topn, m = a.m;
  const long long slice = logical / a.tiles;
  const int t0 = (int)(logical % a.tiles) * T;
  // wave index as a scalar: every per-wave decision below (which sub-tiles
  // take part in a chunk, masking) is then a scalar branch, so no MFMA ever
  // sits under an EXEC-masked region
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int tw = t0 + 32 * w;   // first query of this wave

  const size_t sbase = (size_t)slice * N * D;
  const uint16_t* qs = a.q + sbase;
  const uint16_t* ks = a.k + sbase;
  const uint16_t* vs = a.v + sbase;
  const float c = a.scale_log2;

  // B operands of S^T = K Q^T: Q[query ts + lr][32*kk + 8*lg + e]
  bf16x8 qf[2][KK];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[s][kk] = *reinterpret_cast<const bf16x8*>(qs + (size_t)(tw + 16 * s + lr) * D + 32 * kk + 8 * lg);

  // chunk plan: selected-branch chunks (per query-block group), then window chunks
  const int nB = n * B;
  const int groups = B >= T ? 1 : T / B;
  const int cpg = (nB + 63) / 64;
  const int c_sel = groups * cpg;
  const int lo_off = a.window / 2, hi_off = a.window - a.window / 2;
  const int wlo = max(0, t0 - lo_off);
  const int whi = (int)min((long long)N, (long long)t0 + T - 1 + hi_off);
  const int c_all = c_sel + (whi - wlo + 63) / 64;
  const int blk0 = t0 / B;
  const int lb = 31 - __builtin_clz(B);   // block = 2^lb
  // The score bounds' loads that need no selection table (the precomputed
  // selected-branch bound and the window's block norms) are issued before the
  // table is filled, so their latency overlaps its loads and barrier.
  float ks_pre[2] = {0.f, 0.f}, kl_pre[2] = {0.f, 0.f};
  if (a.knorm) {
    const float* kn = a.knorm + (size_t)slice * m;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ts = tw + 16 * s;   // the sub-tile's query range is uniform
      if (a.selmax) ks_pre[s] = a.selmax[(size_t)slice * m + (ts >> lb)];   // a sub-tile lies in one block
      const int ulo = max(0, ts - lo_off);
      const int uhi = (int)min((long long)N, (long long)ts + 15 + hi_off);
      for (int bl = ulo >> lb; bl <= (uhi - 1) >> lb; ++bl) kl_pre[s] = fmaxf(kl_pre[s], kn[bl]);
    }
  }
  {
    // the selection rows of this tile's query blocks, clamped so that a bad
    // index can never address outside the slice
    const int32_t* selbase = a.sel + ((size_t)slice * m + blk0) * n;
    for (int e = threadIdx.x; e < groups * n; e += 64 * WAVES) {
      const int j = selbase[e];
      SelT[e] = j < 0 ? 0 : (j >= m ? m - 1 : j);
    }
    __syncthreads();
  }

  // Score bounds from the largest key norm of each key block: a query's
  // scaled scores over a set of blocks lie within +-M, M = c*|q|*max|k|
  // (Cauchy-Schwarz).  When every such bound of the wave's queries is at
  // most kBoundMax, each branch's reference is its bound from the start:
  // weights stay at or below about 1, the best one at or above 2^-2M, and
  // no running maximum or rescaling is needed.  Otherwise the lazy running
  // maximum is used.
  float m_sel[2] = {0.f, 0.f}, m_loc[2] = {0.f, 0.f};
  bool bounded = false;
  if (a.knorm) {
    const float* kn = a.knorm + (size_t)slice * m;
    bool ok = true;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float q2 = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(qf[s][kk][e]);
          q2 = fmaf(x, x, q2);
        }
      q2 += __shfl_xor(q2, 16);
      q2 += __shfl_xor(q2, 32);
      const float qn = sqrtf(q2);
      const int ts = tw + 16 * s;
      float ks = ks_pre[s];
      const float kl = kl_pre[s];
      if (!a.selmax) {   // gathered from the selection table
        for (int gi = (ts >> lb) - blk0; gi <= ((ts + 15) >> lb) - blk0; ++gi)
          for (int j = 0; j < n; ++j) ks = fmaxf(ks, kn[SelT[gi * n + j]]);
      }
      m_sel[s] = c * qn * ks;
      m_loc[s] = c * qn * kl;
      ok = ok && m_sel[s] <= kBoundMax && m_loc[s] <= kBoundMax;
    }
    bounded = !__ballot(!ok);
  }

  auto token_of = [&](int ci, int kappa) __attribute__((always_inline)) -> int {
    if (ci < c_sel) {
      const int gi = ci / cpg;
      const int vk = (ci - gi * cpg) * 64 + kappa;
      if (vk >= nB) return -1;
      return SelT[gi * n + vk / B] * B + vk % B;
    }
    const int u = wlo + (ci - c_sel) * 64 + kappa;
    return u < whi ? u : -1;
  };

  // Direct global -> LDS loads of chunk ci: lane l of a 1 KB load writes
  // physical chunk l % CPR of row RPG*grp + l / CPR, which holds logical
  // chunk (l % CPR) ^ swz(row) of that key row.  When the chunk's keys are
  // consecutive tokens tok0 .. tok0+valid-1 (every window chunk, and every
  // selected chunk when a key block holds >= 64 tokens) the per-lane offsets
  // are fixed; otherwise each row looks its token up.
  constexpr int LPW = GPC / WAVES;   // 1 KB loads per tensor per wave
  int lane_off[LPW], lane_row[LPW];
#pragma unroll
  for (int gg = 0; gg < LPW; ++gg) {
    const int grp = w + WAVES * gg;
    lane_row[gg] = RPG * grp + lane / CPR;
    lane_off[gg] = lane_row[gg] * D + 8 * ((lane % CPR) ^ swz<D>(lane_row[gg]));
  }
  // Whole chunks go through buffer loads of the slice's K and V: the
  // per-lane byte offsets are fixed registers and the chunk start is a
  // scalar offset, so issuing a chunk costs no vector instructions.  Byte
  // offsets are 32-bit, hence only for slices under 2 GiB.
  const bool use_rsrc = (long long)N * D * 2 < 0x7fffffffLL;
  const int slice_bytes = use_rsrc ? N * D * 2 : 0;
  const int32x4 rk = slice_rsrc(ks, slice_bytes);
  const int32x4 rv = slice_rsrc(vs, slice_bytes);
  // LDS byte address of this wave's first 1 KB load into K0; load gg of
  // buffer pair P lands (4*P + 2*tensor) * 64*D + gg*WAVES*1024 bytes further
  const int lds_base = lds_addr(KVb) + w * 1024;
  // byte offset of load gg of tensor TS (0 = K, 1 = V) of buffer pair P
  auto at = [](auto P, int TS, auto gg) constexpr { return (2 * decltype(P)::value + TS) * 64 * D * 2 + decltype(gg)::value * WAVES * 1024; };
  auto issue_rows = [&](int tok0, int valid, auto P) __attribute__((always_inline)) {
    if (valid >= 64 && use_rsrc) {   // whole chunk of consecutive tokens: no per-lane checks
      const int soff = __builtin_amdgcn_readfirstlane(tok0 * (D * 2));   // uniform by construction
      static_for<0, LPW>([&](auto gg) __attribute__((always_inline)) {
        dma_buffer_pair_at<at(P, 0, gg), at(P, 1, gg)>(lds_base, 2 * lane_off[gg], rk, rv, soff);
      });
      return;
    }
    const char* kbase = reinterpret_cast<const char*>(ks + (size_t)tok0 * D);   // uniform
    const char* vbase = reinterpret_cast<const char*>(vs + (size_t)tok0 * D);
    static_for<0, LPW>([&](auto gg) __attribute__((always_inline)) {
      const bool ok = lane_row[gg] < valid;
      const unsigned off = 2u * (unsigned)lane_off[gg];
      dma_global_pair_at<at(P, 0, gg), at(P, 1, gg)>(lds_base, ok ? (const void*)(kbase + off) : (const void*)&kZero16,
                                                    ok ? (const void*)(vbase + off) : (const void*)&kZero16);
    });
  };
  auto issue_gather = [&](int ci, auto P) __attribute__((always_inline)) {
    static_for<0, LPW>([&](auto gg) __attribute__((always_inline)) {
      const int row = lane_row[gg];
      const int lc = (lane % CPR) ^ swz<D>(row);
      const int tok = token_of(ci, row);
      dma_global_pair_at<at(P, 0, gg), at(P, 1, gg)>(
          lds_base, tok >= 0 ? (const void*)(ks + (size_t)tok * D + 8 * lc) : (const void*)&kZero16,
          tok >= 0 ? (const void*)(vs + (size_t)tok * D + 8 * lc) : (const void*)&kZero16);
    });
  };
  // loads of chunk ci into buffer pair P (std::integral_constant 0 or 1)
  auto issue = [&](int ci, auto P) __attribute__((always_inline)) {
    if (ci >= c_sel) {
      const int u0 = wlo + (ci - c_sel) * 64;
      issue_rows(u0, whi - u0, P);
    } else if (B >= 64) {   // one group: 128-query tiles only come with blocks of >= 128
      const int vk0 = ci * 64;   // a multiple of 64 inside one key block
      issue_rows((SelT[vk0 >> lb] << lb) + (vk0 & (B - 1)), nB - vk0, P);
    } else {
      issue_gather(ci, P);
    }
  };
  constexpr std::integral_constant<int, 0> P0{};
  constexpr std::integral_constant<int, 1> P1{};

  Branch<D> br[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    branch_init(br[s]);
    if (bounded) br[s].m = m_sel[s] / c;
  }
  float4 pre[2][DT];   // g_CG*o_CG + g_FG*o_FG, formed when the selected branch ends
  // g_L: the 64-query kernel keeps it from the gate row read when the
  // selected branch ends, so its epilogue issues no loads ahead of its
  // stores; the 128-query kernel reads it again in the epilogue.  Each is the
  // faster of the two choices for that kernel, as measured.
  constexpr bool kKeepGL = WAVES == 2;
  float gl[2] = {0.f, 0.f};

  // SAVE: the branch's normalised output and log2-sum-exp m*c + log2(l) of
  // this lane's query, for a backward pass that then skips recomputing them
  // (float32: the backward's D = dO·o must match the weights it recomputes
  // closely, or dQ picks up D's error times the weighted mean key)
  auto save_branch = [&](int s, int which) __attribute__((always_inline)) {
    const int tq = tw + 16 * s + lr;
    const size_t row = (size_t)slice * N + tq;
    const float inv_l = 1.f / br[s].l[0];
    float* dst = a.save_o + (row * 2 + which) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + dt * 16 + 4 * lg) =
          make_float4(br[s].o[dt][0] * inv_l, br[s].o[dt][1] * inv_l, br[s].o[dt][2] * inv_l, br[s].o[dt][3] * inv_l);
    if (lg == 0) a.save_lse[row * 2 + which] = br[s].m * c + log2f(br[s].l[0]);
  };

  auto finish_selected = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (MODE == kSave) save_branch(s, 0);
      const int tq = tw + 16 * s + lr;
      const float* g = a.gates + ((size_t)slice * N + tq) * 3;
      const float g0 = g[0], g1 = g[1] / br[s].l[0];
      if constexpr (kKeepGL) gl[s] = g[2];
      const float* ocg = a.o_cg + ((size_t)slice * m + tq / B) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float4 cg = *reinterpret_cast<const float4*>(ocg + dt * 16 + 4 * lg);
        pre[s][dt] = make_float4(g0 * cg.x + g1 * br[s].o[dt][0], g0 * cg.y + g1 * br[s].o[dt][1],
                                 g0 * cg.z + g1 * br[s].o[dt][2], g0 * cg.w + g1 * br[s].o[dt][3]);
      }
      branch_init(br[s]);
    }
  };

  const float lazy_raw = kLazy / c;
  // BND (std::true_type or std::false_type): whether the wave's references
  // are its score bounds; the chunk code is compiled for each case
  auto step_selected = [&](int ci, const uint16_t* kb, const uint16_t* vb, auto BND) __attribute__((always_inline)) {
    constexpr bool bnd = decltype(BND)::value;
    if (B >= T && nB - ci * 64 >= 64) {   // one group: chunk ci starts at virtual key 64*ci
      attend_full<D, false, bnd>(kb, vb, qf, br, c, lazy_raw, kNoRange, kNoRange);
      return;
    }
    const int gi = groups == 1 ? 0 : ci / cpg;
    const int vc0 = (ci - gi * cpg) * 64;
    bool act[2], msk[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      act[s] = B >= T || (tw + 16 * s) / B == blk0 + gi;
      msk[s] = nB - vc0 < 64;
    }
    attend_chunk<D, bnd>(kb, vb, qf, br, act, msk, c, lazy_raw, [&](int, int kappa) { return vc0 + kappa < nB; });
  };
  auto step_local = [&](int ci, const uint16_t* kb, const uint16_t* vb, auto BND) __attribute__((always_inline)) {
    constexpr bool bnd = decltype(BND)::value;
    const int u0 = wlo + (ci - c_sel) * 64;
    bool act[2], msk[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ts = tw + 16 * s;
      const int ulo = max(0, ts - lo_off);                                  // union of the windows
      const int uhi = (int)min((long long)N, (long long)ts + 15 + hi_off);
      const int ilo = max(0, ts + 15 - lo_off);                             // their intersection
      const int ihi = (int)min((long long)N, (long long)ts + hi_off);
      act[s] = u0 < uhi && u0 + 64 > ulo;
      msk[s] = !(u0 >= ilo && u0 + 64 <= ihi);
    }
    if (act[0] && act[1] && !msk[0] && !msk[1]) {
      attend_full<D, false, bnd>(kb, vb, qf, br, c, lazy_raw, kNoRange, kNoRange);
      return;
    }
    if (act[0] && act[1]) {   // edge of the windows: this lane's query keeps [lo, lo + span)
      int lo[2], span[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int t = tw + 16 * s + lr;
        lo[s] = t - lo_off - u0;
        span[s] = max(0, (int)min((long long)N, (long long)t + hi_off) - u0 - lo[s]);
      }
      attend_full<D, true, bnd>(kb, vb, qf, br, c, lazy_raw, lo, span);
      return;
    }
    attend_chunk<D, bnd>(kb, vb, qf, br, act, msk, c, lazy_raw, [&](int s, int kappa) {
      const int u = u0 + kappa, t = tw + 16 * s + lr;
      return u >= t - lo_off && u < t + hi_off && u < N;
    });
  };

  // Chunks [c0, c1) double-buffered: the loads of chunk ci+1 run while chunk
  // ci is computed; each barrier follows the wave's wait for its own loads.
  auto run = [&](int c0, int c1, auto step, auto BND) __attribute__((always_inline)) {
    if (c0 >= c1) return;
    issue(c0, P0);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __syncthreads();
    for (int ci = c0; ci < c1; ci += 2) {
      if (ci + 1 < c1) issue(ci + 1, P1);
      step(ci, Kb0, Vb0, BND);
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __syncthreads();
      if (ci + 1 >= c1) break;
      if (ci + 2 < c1) issue(ci + 2, P0);
      step(ci + 1, Kb1, Vb1, BND);
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __syncthreads();
    }
  };
  auto branches = [&](auto BND) __attribute__((always_inline)) {
    run(0, c_sel, step_selected, BND);
    finish_selected();
    if constexpr (decltype(BND)::value) {
#pragma unroll
      for (int s = 0; s < 2; ++s) br[s].m = m_loc[s] / c;
    }
    run(c_sel, c_all, step_local, BND);
  };
  if (bounded)
    branches(std::true_type{});
  else
    branches(std::false_type{});

  // gated sum: pre + g_L * o_L
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if constexpr (MODE == kSave) save_branch(s, 1);
    const int tq = tw + 16 * s + lr;
    const float g2 = (kKeepGL ? gl[s] : a.gates[((size_t)slice * N + tq) * 3 + 2]) / br[s].l[0];
    float* dst = a.out + ((size_t)slice * N + tq) * D;
    uint16_t* dstb = nullptr;
    if constexpr (MODE == kMerged) {
      const long long bi = slice / a.heads, h = slice % a.heads;
      dstb = a.out_merged + (((size_t)bi * N + tq) * a.heads + h) * D;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float4 r = pre[s][dt];
      r.x += g2 * br[s].o[dt][0];
      r.y += g2 * br[s].o[dt][1];
      r.z += g2 * br[s].o[dt][2];
      r.w += g2 * br[s].o[dt][3];
      if constexpr (MODE == kMerged) {
        ushort4 o;
        o.x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r.x));
        o.y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r.y));
        o.z = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r.z));
        o.w = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r.w));
        *reinterpret_cast<ushort4*>(dstb + dt * 16 + 4 * lg) = o;
      } else {
        *reinterpret_cast<float4*>(dst + dt * 16 + 4 * lg) = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Any block size and top-n: one wave per query.
//
// The tiled kernel above needs blocks of at least 16 tokens (a 16-query
// sub-tile then lies inside one query block) and a tile's selection rows
// within its 256-entry LDS table.  This kernel covers every other shape
// (blocks of 1 or 4 tokens, or more selected blocks than the table holds).
// A wave owns one query t.  Each branch streams its key list 64 keys at a
// time: lane l forms the float32 score of key l of the group (the query in
// LDS, the key row read whole), the wave takes the group maximum and
// rescales its running sums, and lane d accumulates output dimension d
// while each key's weight and token are broadcast from the lane that formed
// them.  Weights stay float32 (no bf16 rounding).  The selected branch's
// keys are the tokens of the blocks sel[t / block] in listed order, the
// local branch's the clipped centred window; the epilogue is the gated sum
// (and, as in the tiled kernel, the SAVE and MERGED outputs).
__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int D, int MODE>
__global__ __launch_bounds__(256) void fine_generic_kernel(FineArgs a) {
  __shared__ float Qs[4][D];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const long long gq = (long long)blockIdx.x * 4 + w;   // slice * N + t
  if (gq >= a.groups) return;   // whole waves only; no workgroup barrier below
  const int N = a.n_tok, B = a.block, n = a.topn, m = a.m;
  const long long slice = gq / N;
  const int t = (int)(gq % N);
  const int lb = 31 - __builtin_clz(B);
  const uint16_t* ks = a.k + (size_t)slice * N * D;
  const uint16_t* vs = a.v + (size_t)slice * N * D;
  if (lane < D) Qs[w][lane] = bf16_to_f32(a.q[(size_t)gq * D + lane]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float c = a.scale_log2;

  struct Acc {
    float o, l, m;   // lane's output dimension, lane's share of the denominator, running max (log2 units)
  };
  // one branch over `count` keys, key v of the list being token tok(v)
  auto attend = [&](int count, auto tok) __attribute__((always_inline)) -> Acc {
    Acc r{0.f, 0.f, -INFINITY};
    for (int base = 0; base < count; base += kWave) {
      const int v = base + lane;
      const int u = v < count ? tok(v) : -1;
      float sc = -INFINITY;
      if (u >= 0) {
        const uint4* kr = reinterpret_cast<const uint4*>(ks + (size_t)u * D);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D / 8; ++e) {
          const uint4 x = kr[e];
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc = fmaf(Qs[w][8 * e + 2 * h], __uint_as_float(xs[h] << 16), acc);
            acc = fmaf(Qs[w][8 * e + 2 * h + 1], __uint_as_float(xs[h] & 0xffff0000u), acc);
          }
        }
        sc = acc * c;
      }
      const float mn = fmaxf(r.m, wave_max_f32(sc));   // finite: the group's first key is valid
      const float alpha = __builtin_amdgcn_exp2f(r.m - mn);   // 0 while r.m = -inf
      r.o *= alpha;
      r.l *= alpha;
      r.m = mn;
      const float p = u >= 0 ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
      r.l += p;
      const int cnt = min(kWave, count - base);
      for (int jj = 0; jj < cnt; ++jj) {
        const float pj = __shfl(p, jj);
        const int uj = __shfl(u, jj);
        if (lane < D) r.o = fmaf(pj, bf16_to_f32(vs[(size_t)uj * D + lane]), r.o);
      }
    }
    r.l = wave_sum_f32(r.l);
    return r;
  };

  const int blk = t >> lb;
  const int32_t* selrow = a.sel + ((size_t)slice * m + blk) * n;
  const Acc fg = attend(n << lb, [&](int v) __attribute__((always_inline)) {
    int j = selrow[v >> lb];
    j = j < 0 ? 0 : (j >= m ? m - 1 : j);   // a bad index never addresses outside the slice
    return (j << lb) + (v & (B - 1));
  });
  const int lo = max(0, t - a.window / 2);
  const int hi = (int)min((long long)N, (long long)t + (a.window - a.window / 2));
  const Acc lc = attend(hi - lo, [&](int v) __attribute__((always_inline)) { return lo + v; });

  const size_t row = (size_t)gq;
  if constexpr (MODE == kSave) {
    if (lane < D) {
      a.save_o[(row * 2 + 0) * D + lane] = fg.o / fg.l;
      a.save_o[(row * 2 + 1) * D + lane] = lc.o / lc.l;
    }
    if (lane == 0) {
      a.save_lse[row * 2 + 0] = fg.m + log2f(fg.l);
      a.save_lse[row * 2 + 1] = lc.m + log2f(lc.l);
    }
  }
  if (lane < D) {
    const float* g = a.gates + row * 3;
    const float r = g[0] * a.o_cg[((size_t)slice * m + blk) * D + lane] + g[1] * (fg.o / fg.l) +
                    g[2] * (lc.o / lc.l);
    if constexpr (MODE == kMerged) {
      const long long bi = slice / a.heads, h = slice % a.heads;
      a.out_merged[(((size_t)bi * N + t) * a.heads + h) * D + lane] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
    } else {
      a.out[row * D + lane] = r;
    }
  }
}

template <int D>
hipError_t launch_generic(FineArgs a, long long slices, hipStream_t stream) {
  a.groups = slices * a.n_tok;   // queries, four per workgroup
  const dim3 grid((unsigned)((a.groups + 3) / 4));
  if (a.save_o)
    hipLaunchKernelGGL((fine_generic_kernel<D, kSave>), grid, dim3(256), 0, stream, a);
  else if (a.out_merged)
    hipLaunchKernelGGL((fine_generic_kernel<D, kMerged>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fine_generic_kernel<D, kPlain>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// For each query block, the largest key norm over its selected blocks (the
// same clamped indices and the same maximum the fine kernel's prologue would
// form from the selection table), one thread per row.
__global__ __launch_bounds__(256) void sel_bound_kernel(const int32_t* sel, const float* knorm, float* selmax,
                                                        long long rows, int m, int n) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const float* kn = knorm + (r / m) * m;
  const int32_t* row = sel + r * n;
  float mx = 0.f;
  for (int j = 0; j < n; ++j) {
    const int b = row[j];
    mx = fmaxf(mx, kn[b < 0 ? 0 : (b >= m ? m - 1 : b)]);
  }
  selmax[r] = mx;
}

// One workgroup per tile of 32*WAVES queries of every slice: the tile size
// fixes the tile count and the grid together.
template <int D, int WAVES>
hipError_t launch(FineArgs a, long long slices, hipStream_t stream) {
  a.tiles = a.n_tok / (32 * WAVES);
  a.groups = slices * a.tiles;
  dim3 grid((unsigned)a.groups);
  if (a.save_o)
    hipLaunchKernelGGL((fine_kernel<D, WAVES, kSave>), grid, dim3(64 * WAVES), 0, stream, a);
  else if (a.out_merged)
    hipLaunchKernelGGL((fine_kernel<D, WAVES, kMerged>), grid, dim3(64 * WAVES), 0, stream, a);
  else
    hipLaunchKernelGGL((fine_kernel<D, WAVES, kPlain>), grid, dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Whether launch_fine takes the tiled kernel: blocks of at least 16 tokens and
// the tile's selection rows within its table (T = 128 queries when a block
// holds >= 128 tokens and N allows, else 64).
bool fine_tiled(int n_tok, int block, int topn) {
  const int tile = block >= 128 && n_tok % 128 == 0 ? 128 : 64;
  return block >= 16 && (long long)(block >= tile ? 1 : tile / block) * topn <= kSelTable;
}

hipError_t launch_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gates,
                       const float* o_cg, const int32_t* sel, float* out, long long slices,
                       int n_tok, int head_dim, int block, int topn, int window,
                       hipStream_t stream, const float* knorm, float* save_o, float* save_lse,
                       uint16_t* out_merged, int heads, const float* selmax) {
  FineArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gates = gates;
  a.o_cg = o_cg;
  a.sel = sel;
  a.knorm = knorm;
  a.selmax = knorm ? selmax : nullptr;
  a.out = out;
  a.save_o = save_o;
  a.save_lse = save_lse;
  a.out_merged = out_merged;
  a.heads = heads;
  a.n_tok = n_tok;
  a.block = block;
  a.topn = topn;
  a.window = window;
  a.m = n_tok / block;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  // 128-query tiles when a block holds >= 128 tokens (N is then a multiple of
  // 128), else 64 (N = 12*nside^2 with nside^2 >= block >= 16 is a multiple of 64)
  const bool wide = block >= 128 && n_tok % 128 == 0;   // as in fine_tiled
  // the tiled kernel's selection table holds kSelTable entries: the rows of
  // the tile's T/block query blocks (one row when block >= T)
  if (!fine_tiled(n_tok, block, topn))
    return head_dim == 64 ? launch_generic<64>(a, slices, stream) : launch_generic<32>(a, slices, stream);
  if (head_dim == 64) return wide ? launch<64, 4>(a, slices, stream) : launch<64, 2>(a, slices, stream);
  return wide ? launch<32, 4>(a, slices, stream) : launch<32, 2>(a, slices, stream);
}

hipError_t launch_sel_bound(const int32_t* sel, const float* knorm, float* sel_bound, long long slices, int m,
                            int topn, hipStream_t stream) {
  const long long rows = slices * m;
  hipLaunchKernelGGL(sel_bound_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, sel, knorm,
                     sel_bound, rows, m, topn);
  return hipGetLastError();
}

}  // namespace mosaic
