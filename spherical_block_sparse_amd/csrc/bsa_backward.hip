// Backward of the BSA forward: dq, dk, dv and the gate gradients.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse
// Attention gives the forward (three branches over NESTED blocks, gated
// sum); the same page says the model is trained end to end.  The gradient of
// that forward is taken with the selected block indices held fixed (top-n is
// piecewise constant) and the gradients of the block means spread evenly over
// their blocks.
//
// Every branch is softmax attention o = P V over its own key set, whose
// gradient is dV = P^T dO, dS = P ⊙ (dO V^T - D) with D = rowsum(dO ⊙ o),
// dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).  A gated branch (out += g o)
// takes g·dO.  The kernels form P·g in one exponential: the per-query plane
// holds lse - log2|g|, so exp2(S c - that) = P |g|; the gate's sign is folded
// into the bf16 dO of the branch (an exact sign flip, one copy per branch),
// and the score-MFMA for dP starts from -sign(g)·(dO_b·o) instead of zero, so
// that dS = P|g| (sign(g) dO_b V^T - sign(g) dO_b·o) takes one multiply.
// Launch order:
//   1. pool and compressed forward (the forward's kernels) recompute q̄, k̄,
//      v̄ and o_CG;
//   2. prep: dO to bf16 (one copy per fine branch, signed by its gate),
//      do_CG_i = sum over block i of g_CG·dO, the g_CG
//      gradient dO·o_CG, bf16 copies of q̄, k̄, v̄ and do_CG;
//   3. the compressed branch is dense attention over the m pooled rows, so it
//      runs through the same two kernels as the local branch with a window
//      that covers every row (unit gates, upstream gradient do_CG) and gives
//      dq̄, dk̄, dv̄;
//   4. dq kernel (query-major, tiles of 64 queries as in the forward): per
//      branch a forward pass over the branch's key chunks (o, log-sum-exp,
//      dO_b·o, the gate gradient) and a backward pass (P from the
//      log-sum-exp, dP = dO V^T, dS, dQ^T += K^T dS^T); dq̄/B is added in
//      the epilogue;
//   5. the inverted selection (key block -> query blocks that chose it),
//      built per slice with counts, a scan and a sort of each list, so the
//      order of accumulation is fixed;
//   6. dk/dv kernel (key-major, tiles of 64 keys held in registers): the
//      query chunks of the query blocks that selected the tile's block, then
//      the queries whose windows reach the tile; dk̄/B, dv̄/B are added in
//      the epilogue.
// MFMA v_mfma_f32_16x16x32_bf16 throughout, with the forward's LDS layout
// (XOR-swizzled 16-byte chunks) and its transposing reads for the operands
// that contract over rows.  Supported: head_dim 32 or 64, block >= 64, and
// N and m = N/block multiples of 64.
#include "bsa_common.h"

#include <climits>
#include <math.h>

namespace mosaic {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kWaves = 2;            // waves per workgroup
constexpr int kTile = 64;            // queries (dq) or keys (dk/dv) per workgroup

__device__ __forceinline__ shortx4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

template <int D>
struct Dims {
  static constexpr int KK = D / 32;   // k-steps over d
  static constexpr int DT = D / 16;   // 16-row tiles over d
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int RPG = 64 / CPR;   // rows per 1 KB wave load
  static constexpr int GPC = 64 / RPG;   // 1 KB loads per 64-row tile
  static constexpr int LPW = GPC / kWaves;
};

// XOR swizzle of a row's 16-byte chunks (the forward's layout; period 16 rows)
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return 2 * ((row >> 1) & 3) + ((row >> 3) & 1);
  else return (row >> 2) & 3;
}

// Row operand of a staged [64][D] tile: lane lr + 16*lg holds row 16*rt + lr,
// columns 32*kk + 8*lg .. +7 (the A operand of a product over d).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* buf, int rt, int kk) {
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int row = 16 * rt + lr;
  return *reinterpret_cast<const bf16x8*>(buf + row * D + 8 * ((4 * kk + lg) ^ swz<D>(row)));
}

// Transposed operand of a staged tile for a product over rows: d-rows
// 16*dt .. +15, k-slot 8*lg + e holding tile row 32*j + 16*(e/4) + 4*lg + e%4
// (read with ds_read_b64_tr_b16, as the forward reads V^T).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* buf, int j, int dt) {
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int row = 32 * j + 4 * lg + (lr >> 2);
  const int col = dt * 16 + 4 * (lr & 3);
  const uint16_t* src = buf + row * D + 8 * ((col >> 3) ^ swz<D>(row)) + (col & 7);
  const shortx4 lo = lds_read_tr16(src);
  const shortx4 hi = lds_read_tr16(src + 16 * D);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B operand straight from global memory: row r of a [N][D] bf16 tensor,
// columns 32*kk + 8*lg .. +7
template <int D>
__device__ __forceinline__ bf16x8 global_operand(const uint16_t* base, long long r, int kk) {
  const int lg = (threadIdx.x % kWave) / 16;
  return *reinterpret_cast<const bf16x8*>(base + r * D + 32 * kk + 8 * lg);
}

__device__ const uint4 kZero16B = {0u, 0u, 0u, 0u};

// x rounded to the nearest bf16 value (ties to even), as float
__device__ __forceinline__ float bf16_round(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

// Stage rows r0 .. r0+63 of a [N][D] bf16 tensor (rows >= r0+valid read as
// zeros) into a swizzled LDS tile; each wave issues its share of the loads.
template <int D>
__device__ __forceinline__ void stage_rows(uint16_t* buf, const uint16_t* base, long long r0, int valid, int w) {
  using G = Dims<D>;
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int gg = 0; gg < G::LPW; ++gg) {
    const int grp = w + kWaves * gg;
    const int row = G::RPG * grp + lane / G::CPR;
    const int lc = (lane % G::CPR) ^ swz<D>(row);
    const void* src = row < valid ? (const void*)(base + (r0 + row) * D + 8 * lc) : (const void*)&kZero16B;
    dma_global(buf + grp * 512, src);
  }
}

// Stage the per-query statistics of rows r0 .. r0+63 as three arrays of 64
// floats (lse, D, g) from their [3][N] planes: lane L of wave 0 loads rows
// r0 + 4(L%16) .. +3 of plane L/16.  r0 is a multiple of 4 and the plane
// rows past `valid` either exist or are past N in whole groups of 4, which
// read as zeros (lanes 48..63 fill the unused fourth array with zeros).
__device__ __forceinline__ void stage_stats(float* buf, const float* stats, long long r0, int valid, int n_tok,
                                            int w) {
  if (w != 0) return;
  const int lane = threadIdx.x % kWave, plane = lane / 16, g4 = 4 * (lane % 16);
  const bool ok = plane < 3 && g4 < valid;
  dma_global(buf, ok ? (const void*)(stats + (size_t)plane * n_tok + r0 + g4) : (const void*)&kZero16B);
}

constexpr int wait_vm(int n) { return 0x0F70 | (n & 0xF) | (((n >> 4) & 3) << 14); }

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2: renumber them so that XCD x runs a contiguous run of tiles.
// Neighbouring tiles share window rows and mostly the same selected blocks,
// which then hit in one L2.
__device__ __forceinline__ long long xcd_contiguous(long long b, long long groups) {
  const long long q8 = groups / 8, r8 = groups % 8, xcd = b % 8, k = b / 8;
  return xcd < r8 ? xcd * (q8 + 1) + k : r8 * (q8 + 1) + (xcd - r8) * q8 + k;
}

struct BwdArgs {
  const uint16_t* q;      // bf16 [S][N][D]
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dob;    // bf16 upstream gradient of the selected branch [S][N][D], sign of its gate applied
  const uint16_t* dob_loc;// the same for the local branch (the compressed pass: its pooled dO for both)
  const float* dof;       // the same in fp32 (for D = dO·o)
  const float* gates;     // [S][N][3] (g_CG, g_FG, g_L), or null: unit gates
  const int32_t* sel;     // [S][m][n] selection, or null: no selected branch
  const int32_t* inv_off; // [S][m+1] inverted selection offsets
  const int32_t* inv_list;// [S][m*n] query blocks per key block
  float* stats;           // [2][S][3][N] per branch planes lse - log2|g|, -sign(g) dO_b·o, g; branch 0 selected, 1 local
  float* dq;              // [S][N][D] fp32 out
  float* dk;
  float* dv;
  float* dgates;          // [S][N][3] out (columns 1, 2 here), or null
  const float* addq;      // pooled gradients added with weight 1/block, or null
  const float* addk;
  const float* addv;
  int n_tok;
  int block;              // selection block (selected branch) and pooled-gradient block
  int topn;
  int window;
  int m;
  long long slices;
  float scale_log2;       // log2(e) / sqrt(d)
  float inv_sqrt_d;
};

// ---------------------------------------------------------------------------
// dq kernel: 64 queries per workgroup, 2 waves x 2 sub-tiles of 16 queries.

template <int D>
struct SubState {
  floatx4 o[Dims<D>::DT];   // O^T (pass 1) for query lr, d = 16*dt + 4*lg + i
  floatx4 l;                // denominator (ones MFMA: every entry the row sum)
  float m;                  // running max, raw units
};

template <int D, bool SEL, bool PASS1>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
  using G = Dims<D>;
  constexpr int KK = G::KK, DT = G::DT;
  __shared__ __attribute__((aligned(16))) uint16_t KV[4 * 64 * D];   // K0, V0, K1, V1
  __shared__ int SelT[64];
  const int N = a.n_tok, B = a.block, n = a.topn;
  const int tiles = N / kTile;
  const long long tile = xcd_contiguous(blockIdx.x, gridDim.x);
  const long long slice = tile / tiles;
  const int t0 = (int)(tile % tiles) * kTile;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int tw = t0 + 32 * w;
  const size_t sb = (size_t)slice * N * D;
  const uint16_t *qs = a.q + sb, *ks = a.k + sb, *vs = a.v + sb;
  const float* dofs = a.dof + sb;
  const float c = a.scale_log2;

  // q operands; dO operands per branch (each branch's dO carries the sign of its gate)
  bf16x8 qf[2][KK], df[2][KK];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[s][kk] = global_operand<D>(qs, tw + 16 * s + lr, kk);
  floatx4 dqa[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqa[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int m = a.m;
  if constexpr (SEL) {
    const int32_t* row = a.sel + ((size_t)slice * m + t0 / B) * n;
    for (int e = threadIdx.x; e < n; e += 64 * kWaves) {
      const int j = row[e];
      SelT[e] = j < 0 ? 0 : (j >= m ? m - 1 : j);
    }
  }
  __syncthreads();

  const int lo_off = a.window / 2, hi_off = a.window - a.window / 2;
  // buffer pair p: K at KV + 2p*64*D, V right after it
  auto Kb = [&](int p) __attribute__((always_inline)) { return KV + (p ? 2 * 64 * D : 0); };
  auto Vb = [&](int p) __attribute__((always_inline)) { return KV + (p ? 3 * 64 * D : 64 * D); };

  // one branch: chunks [0, nc); first token and valid count of chunk ci,
  // whether its scores need the per-lane key range, and that range
  auto branch = [&](int br_id, int nc, auto chunk_tok, auto chunk_valid) __attribute__((always_inline)) {
    float g[2];
    const uint16_t* dos = (br_id == 0 ? a.dob : a.dob_loc) + sb;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int t = tw + 16 * s + lr;
      g[s] = a.gates ? a.gates[((size_t)slice * N + t) * 3 + 1 + br_id] : 1.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) df[s][kk] = global_operand<D>(dos, t, kk);
    }
    // key range of this lane's query in chunk ci (all keys for the selected branch)
    auto range = [&](int ci, int s, int& lo, int& span) __attribute__((always_inline)) -> bool {
      if (br_id == 0) { lo = 0; span = 64; return false; }
      const int u0 = chunk_tok(ci);
      const int t = tw + 16 * s + lr;
      lo = t - lo_off - u0;
      span = max(0, min(N, t + hi_off) - u0 - lo);
      const int ts = tw + 16 * s;   // the sub-tile's windows all contain the chunk?
      const int ilo = max(0, ts + 15 - lo_off), ihi = min(N, ts + hi_off);
      return !(u0 >= ilo && u0 + 64 <= ihi);
    };
    auto scores = [&](const uint16_t* kb, floatx4 (&acc)[2][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[s][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = row_operand<D>(kb, kt, kk);
#pragma unroll
          for (int s = 0; s < 2; ++s)
            acc[s][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s][kk], acc[s][kt], 0, 0, 0);
        }
    };
    auto mask = [&](int ci, floatx4 (&acc)[2][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        int lo, span;
        if (!range(ci, s, lo, span)) continue;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((unsigned)(16 * kt + 4 * lg + i - lo) >= (unsigned)span) acc[s][kt][i] = -INFINITY;
      }
    };
    // double-buffered chunk loop: loads of chunk ci+1 run while ci is computed
    auto sweep = [&](auto step) __attribute__((always_inline)) {
      stage_rows<D>(Kb(0), ks, chunk_tok(0), chunk_valid(0), w);
      stage_rows<D>(Vb(0), vs, chunk_tok(0), chunk_valid(0), w);
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __syncthreads();
      for (int ci = 0; ci < nc; ++ci) {
        const int p = ci & 1;
        if (ci + 1 < nc) {
          stage_rows<D>(Kb(p ^ 1), ks, chunk_tok(ci + 1), chunk_valid(ci + 1), w);
          stage_rows<D>(Vb(p ^ 1), vs, chunk_tok(ci + 1), chunk_valid(ci + 1), w);
        }
        step(ci, Kb(p), Vb(p));
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        __syncthreads();
      }
    };

    float lse[2], dsub[2];
    if constexpr (PASS1) {
      // pass 1: forward (online softmax) for o, the log-sum-exp and D
      SubState<D> st[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st[s].o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        st[s].l = floatx4{0.f, 0.f, 0.f, 0.f};
        st[s].m = -INFINITY;
      }
      bf16x8 ones;
#pragma unroll
      for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);
      sweep([&](int ci, const uint16_t* kb, const uint16_t* vb) __attribute__((always_inline)) {
        floatx4 acc[2][4];
        scores(kb, acc);
        mask(ci, acc);
        bf16x8 pb[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float mx = acc[s][0][0];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[s][kt][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mnew = fmaxf(st[s].m, mx);
          const float alpha = st[s].m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st[s].m - mnew) * c);
          st[s].m = mnew;
          st[s].l *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) st[s].o[dt] *= alpha;
          const float nmc = mnew == -INFINITY ? 0.f : -mnew * c;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pb[s][kt >> 1][4 * (kt & 1) + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(acc[s][kt][i], c, nmc)));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int s = 0; s < 2; ++s) st[s].l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[s][j], st[s].l, 0, 0, 0);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 va = tr_operand<D>(vb, j, dt);
#pragma unroll
            for (int s = 0; s < 2; ++s) st[s].o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[s][j], st[s].o[dt], 0, 0, 0);
          }
        }
      });
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int t = tw + 16 * s + lr;
        const float inv_l = 1.f / st[s].l[0];
        // dg = dO·o (the gate gradient) with dO in float32; dO_b·o with the
        // bf16 dO_b that dP = dO_b V^T uses, so that sum_u dS_u stays zero up
        // to rounding (otherwise dO's rounding error, times the mean key,
        // lands in every dQ)
        float dg = 0.f, dgb = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float4 d4 = *reinterpret_cast<const float4*>(dofs + (size_t)t * D + dt * 16 + 4 * lg);
          dg += d4.x * st[s].o[dt][0] + d4.y * st[s].o[dt][1] + d4.z * st[s].o[dt][2] + d4.w * st[s].o[dt][3];
          dgb += bf16_round(d4.x) * st[s].o[dt][0] + bf16_round(d4.y) * st[s].o[dt][1] +
                 bf16_round(d4.z) * st[s].o[dt][2] + bf16_round(d4.w) * st[s].o[dt][3];
        }
        dg *= inv_l;
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
        dgb *= inv_l;
        dgb += __shfl_xor(dgb, 16);
        dgb += __shfl_xor(dgb, 32);
        // the planes of the kernels' product form: P|g| = exp2(S c - lse + log2|g|),
        // dS = P|g| (sign(g) dP - sign(g) dO_b·o); |g| = 0 gives an exponent of -inf
        lse[s] = st[s].m * c + log2f(st[s].l[0]) - log2f(fabsf(g[s]));
        dsub[s] = signbit(g[s]) ? dgb : -dgb;
        if (lg == 0) {
          float* sp = a.stats + ((size_t)br_id * a.slices + slice) * 3 * N + t;
          sp[0] = lse[s];
          sp[N] = dsub[s];
          sp[2 * N] = g[s];
          if (a.dgates) a.dgates[((size_t)slice * N + t) * 3 + 1 + br_id] = dg;
        }
      }
    } else {   // the training forward saved lse; the prep kernel formed the planes and dgates
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float* sp = a.stats + ((size_t)br_id * a.slices + slice) * 3 * N + tw + 16 * s + lr;
        lse[s] = sp[0];
        dsub[s] = sp[N];
      }
    }

    // pass 2: dS from the log-sum-exp, dQ^T += K^T dS^T
    sweep([&](int ci, const uint16_t* kb, const uint16_t* vb) __attribute__((always_inline)) {
      floatx4 acc[2][4], dpa[2][4];
      scores(kb, acc);
      mask(ci, acc);
      // dP starts from -sign(g) dO_b·o, so the MFMAs leave sign(g) dP - sign(g) dO_b·o
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) dpa[s][kt] = floatx4{dsub[s], dsub[s], dsub[s], dsub[s]};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 va = row_operand<D>(vb, kt, kk);
#pragma unroll
          for (int s = 0; s < 2; ++s)
            dpa[s][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, df[s][kk], dpa[s][kt], 0, 0, 0);
        }
      bf16x8 ds[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pg = __builtin_amdgcn_exp2f(fmaf(acc[s][kt][i], c, -lse[s]));   // P |g|
            ds[s][kt >> 1][4 * (kt & 1) + i] = static_cast<__bf16>(pg * dpa[s][kt][i]);
          }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 ka = tr_operand<D>(kb, j, dt);
#pragma unroll
          for (int s = 0; s < 2; ++s) dqa[s][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ds[s][j], dqa[s][dt], 0, 0, 0);
        }
    });
  };

  if constexpr (SEL) {
    const int lb = 31 - __builtin_clz(B);
    const int nc = n * B / 64;
    branch(0, nc, [&](int ci) { const int vk0 = ci * 64; return (SelT[vk0 >> lb] << lb) + (vk0 & (B - 1)); },
           [&](int) { return 64; });
  }
  {
    const int wlo = max(0, t0 - lo_off);
    const int whi = min(N, t0 + kTile - 1 + hi_off);
    const int nc = (whi - wlo + 63) / 64;
    branch(1, nc, [&](int ci) { return wlo + ci * 64; }, [&](int ci) { return min(64, whi - wlo - ci * 64); });
  }

  // epilogue: dq = dQ^T / sqrt(d) (+ the pooled gradient / block).  The
  // pooled rows are all loaded before the first store: the compiler cannot
  // rule out that they alias dq, so a load written after a store stays
  // behind it, latency exposed.
  float4 addp[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = tw + 16 * s + lr;
    const float* add = a.addq ? a.addq + ((size_t)slice * m + t / B) * D : nullptr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      addp[s][dt] = add ? *reinterpret_cast<const float4*>(add + dt * 16 + 4 * lg) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = tw + 16 * s + lr;
    float* dst = a.dq + sb + (size_t)t * D;
    const float ab = 1.f / B;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float4 r = make_float4(dqa[s][dt][0] * a.inv_sqrt_d, dqa[s][dt][1] * a.inv_sqrt_d,
                             dqa[s][dt][2] * a.inv_sqrt_d, dqa[s][dt][3] * a.inv_sqrt_d);
      if (a.addq) {
        const float4 p = addp[s][dt];
        r.x += p.x * ab; r.y += p.y * ab; r.z += p.z * ab; r.w += p.w * ab;
      }
      *reinterpret_cast<float4*>(dst + dt * 16 + 4 * lg) = r;
    }
  }
}

// ---------------------------------------------------------------------------
// dk/dv kernel: 64 keys per workgroup in registers, 2 waves x 2 sub-tiles of
// 16 keys; query chunks of 64 stream through LDS.

template <int D, bool SEL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(BwdArgs a) {
  using G = Dims<D>;
  constexpr int KK = G::KK, DT = G::DT;
  __shared__ __attribute__((aligned(16))) uint16_t QO[4 * 64 * D];   // Q0, dO0, Q1, dO1
  __shared__ __attribute__((aligned(16))) float ST[2][4 * 64];        // per-query lse[64], D[64], g[64]
  const int N = a.n_tok, B = a.block;
  const int tiles = N / kTile;
  const long long tile = xcd_contiguous(blockIdx.x, gridDim.x);
  const long long slice = tile / tiles;
  const int u0 = (int)(tile % tiles) * kTile;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int uw = u0 + 32 * w;
  const size_t sb = (size_t)slice * N * D;
  const uint16_t *qs = a.q + sb, *ks = a.k + sb, *vs = a.v + sb;
  const float c = a.scale_log2;

  bf16x8 kf[2][KK], vf[2][KK];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf[s][kk] = global_operand<D>(ks, uw + 16 * s + lr, kk);
      vf[s][kk] = global_operand<D>(vs, uw + 16 * s + lr, kk);
    }
  floatx4 dka[2][DT], dva[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dka[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      dva[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  // buffer pair p: Q at QO + 2p*64*D, dO right after it
  auto Qb = [&](int p) __attribute__((always_inline)) { return QO + (p ? 2 * 64 * D : 0); };
  auto Ob = [&](int p) __attribute__((always_inline)) { return QO + (p ? 3 * 64 * D : 64 * D); };
  const int lo_off = a.window / 2, hi_off = a.window - a.window / 2;

  // one phase: query chunks [0, nc) with first row chunk_row(ci) and valid
  // count chunk_valid(ci); LOCAL masks by the windows
  auto phase = [&](int br_id, int nc, auto chunk_row, auto chunk_valid, auto local) __attribute__((always_inline)) {
    constexpr bool LOCAL = decltype(local)::value;
    const float* stats = a.stats + ((size_t)br_id * a.slices + slice) * 3 * N;
    const uint16_t* dos = (br_id == 0 ? a.dob : a.dob_loc) + sb;   // the branch's signed dO
    auto stage = [&](int ci, int p) __attribute__((always_inline)) {
      stage_rows<D>(Qb(p), qs, chunk_row(ci), chunk_valid(ci), w);
      stage_rows<D>(Ob(p), dos, chunk_row(ci), chunk_valid(ci), w);
      stage_stats(&ST[p][0], stats, chunk_row(ci), chunk_valid(ci), N, w);
    };
    if (nc <= 0) return;
    stage(0, 0);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __syncthreads();
    for (int ci = 0; ci < nc; ++ci) {
      const int p = ci & 1;
      if (ci + 1 < nc) stage(ci + 1, p ^ 1);
      const uint16_t* qb = Qb(p);
      const uint16_t* ob = Ob(p);
      const float* stt = p ? &ST[1][0] : &ST[0][0];
      const int r0 = chunk_row(ci), nv = chunk_valid(ci);
      // in halves of 32 queries (j): S = Q K^T and dP = dO V^T, where the
      // lane holds key lr of sub-tile s and queries 32*j + 16*h + 4*lg + i;
      // then dV^T += dO^T (P g) and dK^T += Q^T dS over those queries.  dO
      // is the branch's signed copy, and dP starts from the plane
      // -sign(g) dO_b·o, so the MFMAs leave sign(g) dP - sign(g) dO_b·o.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        floatx4 sa[2][2], dpa[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 d4 = *reinterpret_cast<const float4*>(stt + 64 + 32 * j + 16 * h + 4 * lg);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            sa[s][h] = floatx4{0.f, 0.f, 0.f, 0.f};
            dpa[s][h] = floatx4{d4.x, d4.y, d4.z, d4.w};
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 qa = row_operand<D>(qb, 2 * j + h, kk);
            const bf16x8 oa = row_operand<D>(ob, 2 * j + h, kk);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              sa[s][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[s][kk], sa[s][h], 0, 0, 0);
              dpa[s][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[s][kk], dpa[s][h], 0, 0, 0);
            }
          }
        bf16x8 pg[2], ds[2];
        // P|g| = exp2(S c - (lse - log2|g|)) and dS = P|g| (dP - D) from the
        // signed accumulators.  Padded rows and (local phase) keys outside
        // the query's window get exponent -inf; key u is inside the window
        // of query t iff u - t + lo_off < window (unsigned), and u - t is a
        // per-lane base plus a constant.
        const int dbase = uw + lr - r0 - 32 * j - 4 * lg + lo_off;
        const int vbase = nv - 32 * j - 4 * lg;   // row qi valid iff qi - 32j - 4lg < vbase
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q0 = 32 * j + 16 * h + 4 * lg;   // the lane's first query row of the chunk
          const float4 lse4 = *reinterpret_cast<const float4*>(stt + q0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lse = i == 0 ? lse4.x : i == 1 ? lse4.y : i == 2 ? lse4.z : lse4.w;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              float x = fmaf(sa[s][h][i], c, -lse);
              if constexpr (LOCAL) {
                const bool ok = 16 * h + i < vbase && (unsigned)(dbase + 16 * s - 16 * h - i) < (unsigned)a.window;
                x = ok ? x : -INFINITY;
              }
              const float p = __builtin_amdgcn_exp2f(x);   // P |g|
              pg[s][4 * h + i] = static_cast<__bf16>(p);
              ds[s][4 * h + i] = static_cast<__bf16>(p * dpa[s][h][i]);
            }
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 ot = tr_operand<D>(ob, j, dt);
          const bf16x8 qt_ = tr_operand<D>(qb, j, dt);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            dva[s][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ot, pg[s], dva[s][dt], 0, 0, 0);
            dka[s][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt_, ds[s], dka[s][dt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __syncthreads();
    }
  };

  if constexpr (SEL) {
    // query blocks that selected the tile's key block, each B/64 chunks
    const int j = u0 / B;
    const int32_t* off = a.inv_off + (size_t)slice * (a.m + 1);
    const int32_t* lst = a.inv_list + (size_t)slice * a.m * a.topn;
    const int beg = off[j], cnt = off[j + 1] - beg;
    const int per = B / 64;
    phase(0, cnt * per, [&](int ci) { return lst[beg + ci / per] * B + (ci % per) * 64; }, [&](int) { return 64; },
          std::integral_constant<bool, false>{});
  }
  {
    const int tlo = max(0, u0 - hi_off + 1) & ~3;   // a multiple of 4 for the statistics staging
    const int thi = min(N, u0 + kTile + lo_off);
    phase(1, (thi - tlo + 63) / 64, [&](int ci) { return tlo + ci * 64; },
          [&](int ci) { return min(64, thi - tlo - ci * 64); }, std::integral_constant<bool, true>{});
  }

  // epilogue: dk = dK^T / sqrt(d), dv = dV^T (+ pooled gradients / block),
  // every pooled row loaded before the first store (as in the dq kernel)
  const int m = a.m;
  float4 addkp[2][DT], addvp[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int u = uw + 16 * s + lr;
    const float* addk = a.addk ? a.addk + ((size_t)slice * m + u / B) * D : nullptr;
    const float* addv = a.addv ? a.addv + ((size_t)slice * m + u / B) * D : nullptr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      addkp[s][dt] = addk ? *reinterpret_cast<const float4*>(addk + dt * 16 + 4 * lg) : make_float4(0.f, 0.f, 0.f, 0.f);
      addvp[s][dt] = addv ? *reinterpret_cast<const float4*>(addv + dt * 16 + 4 * lg) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int u = uw + 16 * s + lr;
    const float ab = 1.f / B;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float4 rk = make_float4(dka[s][dt][0] * a.inv_sqrt_d, dka[s][dt][1] * a.inv_sqrt_d,
                              dka[s][dt][2] * a.inv_sqrt_d, dka[s][dt][3] * a.inv_sqrt_d);
      float4 rv = make_float4(dva[s][dt][0], dva[s][dt][1], dva[s][dt][2], dva[s][dt][3]);
      if (a.addk) {
        const float4 p = addkp[s][dt];
        rk.x += p.x * ab; rk.y += p.y * ab; rk.z += p.z * ab; rk.w += p.w * ab;
      }
      if (a.addv) {
        const float4 p = addvp[s][dt];
        rv.x += p.x * ab; rv.y += p.y * ab; rv.z += p.z * ab; rv.w += p.w * ab;
      }
      *reinterpret_cast<float4*>(a.dk + sb + (size_t)u * D + dt * 16 + 4 * lg) = rk;
      *reinterpret_cast<float4*>(a.dv + sb + (size_t)u * D + dt * 16 + 4 * lg) = rv;
    }
  }
}

// ---------------------------------------------------------------------------
// prep: one workgroup per (slice, block of B tokens).

struct PrepArgs {
  const float* dout;       // [S][N][D]
  const float* gates;      // [S][N][3]
  const float* o_cg;       // [S][m][D]
  const double* qbar;      // [S][m][D]
  const double* kbar;
  const float* vbar;
  uint16_t* dob;           // out bf16 [S][N][D]: sign(g_FG) dO (the selected branch's)
  uint16_t* dob_loc;       // out bf16 [S][N][D]: sign(g_L) dO (the local branch's)
  float* docg;             // out [S][m][D]
  uint16_t* docg_b;        // out bf16 [S][m][D]
  uint16_t* qbar_b;        // out bf16 [S][m][D]
  uint16_t* kbar_b;
  uint16_t* vbar_b;
  float* dgates;           // out column 0 (or null); with save_o also columns 1, 2
  const float* save_o;     // [S][N][2][D] o_FG, o_L of the training forward, or null
  const float* save_lse;   // [S][N][2]
  float* stats;            // with save_o: out [2][S][3][N] planes lse - log2|g|, -sign(g) dO_b·o, g
  long long slices;
  int n_tok, block, m;
};

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepArgs a) {
  constexpr int C4 = D / 4;                 // float4 columns per row
  constexpr int RS = 256 / C4;              // rows per sweep
  __shared__ float part[RS][D];
  const long long gb = blockIdx.x;          // slice * m + block
  const long long slice = gb / a.m;
  const int blk = (int)(gb % a.m);
  const int x = threadIdx.x, c4 = x % C4, r0 = x / C4;
  const float4 ocg = *reinterpret_cast<const float4*>(a.o_cg + gb * D + 4 * c4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // Rows are taken kBatch sweeps at a time, every load of a batch issued
  // before its first store: the compiler cannot rule out that the outputs
  // alias the inputs, so a load written after a store stays behind it.
  constexpr int kBatch = 4;
  const bool sv = a.save_o != nullptr;
  for (int rb = r0; rb < a.block; rb += kBatch * RS) {
    float4 d4[kBatch], ob[kBatch][2];
    float g[kBatch][3], lse[kBatch][2];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int r = rb + i * RS;
      if (r >= a.block) continue;
      const long long row = slice * a.n_tok + (long long)blk * a.block + r;
      d4[i] = *reinterpret_cast<const float4*>(a.dout + row * D + 4 * c4);
#pragma unroll
      for (int r = 0; r < 3; ++r) g[i][r] = a.gates[row * 3 + r];
      if (sv) {
#pragma unroll
        for (int br = 0; br < 2; ++br) {
          ob[i][br] = *reinterpret_cast<const float4*>(a.save_o + (row * 2 + br) * D + 4 * c4);
          lse[i][br] = a.save_lse[row * 2 + br];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int r = rb + i * RS;
      if (r >= a.block) continue;
      const long long t = (long long)blk * a.block + r;
      const long long row = slice * a.n_tok + t;
      const float4 dv = d4[i];
      const float g0 = g[i][0];
      acc.x += g0 * dv.x; acc.y += g0 * dv.y; acc.z += g0 * dv.z; acc.w += g0 * dv.w;
      // each fine branch's bf16 dO carries the sign of the branch's gate
      // (rounding commutes with the sign, so this is bf16(dO) or its negation)
      ushort4 b;
      b.x = bf16_bits(dv.x); b.y = bf16_bits(dv.y); b.z = bf16_bits(dv.z); b.w = bf16_bits(dv.w);
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        const uint16_t sg = signbit(g[i][1 + br]) ? 0x8000 : 0;
        ushort4 bs;
        bs.x = b.x ^ sg; bs.y = b.y ^ sg; bs.z = b.z ^ sg; bs.w = b.w ^ sg;
        *reinterpret_cast<ushort4*>((br == 0 ? a.dob : a.dob_loc) + row * D + 4 * c4) = bs;
      }
      float dg = dv.x * ocg.x + dv.y * ocg.y + dv.z * ocg.z + dv.w * ocg.w;
#pragma unroll
      for (int sh = 1; sh < C4; sh <<= 1) dg += __shfl_xor(dg, sh);
      if (c4 == 0 && a.dgates) a.dgates[row * 3] = dg;
      if (sv) {   // dg_br = dO·o_br for the selected (0) and local (1) branches
#pragma unroll
        for (int br = 0; br < 2; ++br) {
          // e = dO·o_br for the gate gradient; eb = dO_b·o_br (bf16 dO, as dP
          // uses it) for D, so that the logit gradients of a row sum to zero
          const float4 o4 = ob[i][br];
          float e = dv.x * o4.x + dv.y * o4.y + dv.z * o4.z + dv.w * o4.w;
          float eb = bf16_round(dv.x) * o4.x + bf16_round(dv.y) * o4.y + bf16_round(dv.z) * o4.z +
                     bf16_round(dv.w) * o4.w;
#pragma unroll
          for (int sh = 1; sh < C4; sh <<= 1) {
            e += __shfl_xor(e, sh);
            eb += __shfl_xor(eb, sh);
          }
          if (c4 == 0) {   // the planes of the kernels' product form (see the header)
            const float gb = g[i][1 + br];
            float* sp = a.stats + ((size_t)br * a.slices + slice) * 3 * a.n_tok + t;
            sp[0] = lse[i][br] - log2f(fabsf(gb));
            sp[a.n_tok] = signbit(gb) ? eb : -eb;
            sp[2 * (size_t)a.n_tok] = gb;
            a.dgates[row * 3 + 1 + br] = e;
          }
        }
      }
    }
  }
  part[r0][4 * c4 + 0] = acc.x;
  part[r0][4 * c4 + 1] = acc.y;
  part[r0][4 * c4 + 2] = acc.z;
  part[r0][4 * c4 + 3] = acc.w;
  __syncthreads();
  if (x < D) {
    float sum = 0.f;
    for (int r = 0; r < RS; ++r) sum += part[r][x];
    a.docg[gb * D + x] = sum;
    a.docg_b[gb * D + x] = bf16_bits(sum);
    a.qbar_b[gb * D + x] = bf16_bits((float)a.qbar[gb * D + x]);
    a.kbar_b[gb * D + x] = bf16_bits((float)a.kbar[gb * D + x]);
    a.vbar_b[gb * D + x] = bf16_bits(a.vbar[gb * D + x]);
  }
}

// ---------------------------------------------------------------------------
// inverted selection, one workgroup per slice: off[j] .. off[j+1] indexes
// the ascending list of query blocks whose selection holds key block j.
// Counts and cursors live in LDS (m <= kIndexMaxBlocks); the entries are
// scattered into `tmp` in arrival order.  bwd_list_sort_kernel then
// rank-sorts each list by one wave into `list`, ordered by (query block,
// position in `tmp`), so that the result is deterministic and a permutation
// even if a selection row repeats an index.

constexpr int kIndexThreads = 1024;

__global__ __launch_bounds__(kIndexThreads) void bwd_index_kernel(const int32_t* sel, int32_t* off, int32_t* tmp,
                                                                   int m, int n) {
  __shared__ int32_t cnt[kIndexMaxBlocks + 1];
  __shared__ int32_t wsum[kIndexThreads / 64];
  const long long slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int total = m * n;
  const int32_t* s = sel + slice * total;
  int32_t* o = off + slice * (m + 1);
  int32_t* t = tmp + slice * total;
  for (int j = tid; j < m; j += kIndexThreads) cnt[j] = 0;
  __syncthreads();
  for (int e = tid; e < total; e += kIndexThreads) atomicAdd(&cnt[min(max(s[e], 0), m - 1)], 1);
  __syncthreads();

  // exclusive scan: each thread owns a contiguous run of counts
  const int per = (m + kIndexThreads - 1) / kIndexThreads;
  const int jb = min(tid * per, m), je = min(jb + per, m);
  int run = 0;
  for (int j = jb; j < je; ++j) run += cnt[j];
  int incl = run;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = incl - run;
  for (int x = 0; x < w; ++x) base += wsum[x];
  for (int j = jb; j < je; ++j) {
    const int c = cnt[j];
    cnt[j] = base;
    o[j] = base;
    base += c;
  }
  if (tid == 0) o[m] = total;
  __syncthreads();

  for (int e = tid; e < total; e += kIndexThreads) t[atomicAdd(&cnt[min(max(s[e], 0), m - 1)], 1)] = e / n;
}

// Each inverted list sorted by query block (the scatter above leaves the
// order of its atomics), so that dk/dv accumulate in a fixed order: one wave
// per list over all slices, a rank sort (the element at position p goes to
// the number of elements before it in (value, position) order).
constexpr int kSortWaves = 4;

__global__ __launch_bounds__(64 * kSortWaves) void bwd_list_sort_kernel(const int32_t* off, const int32_t* tmp,
                                                                        int32_t* list, long long lists, int m,
                                                                        int total) {
  const long long id = (long long)blockIdx.x * kSortWaves + threadIdx.x / 64;
  if (id >= lists) return;   // whole waves leave together
  const int lane = threadIdx.x & 63;
  const long long slice = id / m;
  const int j = (int)(id - slice * m);
  const int32_t* o = off + slice * (m + 1);
  const int32_t* t = tmp + slice * total;
  int32_t* l = list + slice * total;
  const int b = o[j], len = o[j + 1] - b;
  for (int pc = 0; pc < len; pc += 64) {
    const int p = pc + lane;
    const int x = p < len ? t[b + p] : INT_MAX;
    int rank = 0;
    for (int qc = 0; qc < len; qc += 64) {
      const int y = qc + lane < len ? t[b + qc + lane] : INT_MAX;
      const int qn = min(64, len - qc);
      for (int r = 0; r < qn; ++r) {   // r is uniform: a scalar broadcast, no LDS permute
        const int yr = __builtin_amdgcn_readlane(y, r);
        rank += (yr < x) || (yr == x && qc + r < p);
      }
    }
    if (p < len) l[b + rank] = x;
  }
}

template <int D>
hipError_t launch_d(const BwdLaunch& L, hipStream_t stream) {
  const long long S = L.slices;
  const int N = L.n_tok, m = L.n_tok / L.block;
  // prep
  PrepArgs p;
  p.dout = L.dout; p.gates = L.gates; p.o_cg = L.o_cg; p.qbar = L.qbar; p.kbar = L.kbar; p.vbar = L.vbar;
  p.dob = L.dob; p.dob_loc = L.dob_loc; p.docg = L.docg; p.docg_b = L.docg_b; p.qbar_b = L.qbar_b; p.kbar_b = L.kbar_b; p.vbar_b = L.vbar_b;
  p.dgates = L.dgates; p.n_tok = N; p.block = L.block; p.m = m;
  p.save_o = L.save_o; p.save_lse = L.save_lse; p.stats = L.stats; p.slices = S;
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)(S * m)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float c = (float)(1.4426950408889634 / sqrt((double)D));
  const float isd = (float)(1.0 / sqrt((double)D));
  // compressed branch: dense attention over the pooled rows (window covers all)
  BwdArgs cg = {};
  cg.q = L.qbar_b; cg.k = L.kbar_b; cg.v = L.vbar_b; cg.dob = L.docg_b; cg.dob_loc = L.docg_b; cg.dof = L.docg;
  cg.gates = nullptr; cg.sel = nullptr; cg.stats = L.stats_cg;
  cg.dq = L.dqbar; cg.dk = L.dkbar; cg.dv = L.dvbar; cg.dgates = nullptr;
  cg.n_tok = m; cg.block = 1; cg.topn = 0; cg.window = 2 * m + 1; cg.m = m; cg.slices = S;
  cg.scale_log2 = c; cg.inv_sqrt_d = isd;
  hipLaunchKernelGGL((bwd_dq_kernel<D, false, true>), dim3((unsigned)(S * (m / kTile))), dim3(64 * kWaves), 0, stream, cg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((unsigned)(S * (m / kTile))), dim3(64 * kWaves), 0, stream, cg);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // fine branches
  if (m > kIndexMaxBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_index_kernel, dim3((unsigned)S), dim3(kIndexThreads), 0, stream, L.sel, L.inv_off,
                     L.inv_tmp, m, L.topn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_list_sort_kernel, dim3((unsigned)((S * m + kSortWaves - 1) / kSortWaves)),
                     dim3(64 * kSortWaves), 0, stream, L.inv_off, L.inv_tmp, L.inv_list, S * m, m, m * L.topn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  BwdArgs f = {};
  f.q = L.q; f.k = L.k; f.v = L.v; f.dob = L.dob; f.dob_loc = L.dob_loc; f.dof = L.dout; f.gates = L.gates; f.sel = L.sel;
  f.inv_off = L.inv_off; f.inv_list = L.inv_list; f.stats = L.stats;
  f.dq = L.dq; f.dk = L.dk; f.dv = L.dv; f.dgates = L.dgates;
  f.addq = L.dqbar; f.addk = L.dkbar; f.addv = L.dvbar;
  f.n_tok = N; f.block = L.block; f.topn = L.topn; f.window = L.window; f.m = m; f.slices = S;
  f.scale_log2 = c; f.inv_sqrt_d = isd;
  if (L.save_o)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, false>), dim3((unsigned)(S * (N / kTile))), dim3(64 * kWaves), 0, stream,
                       f);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), dim3((unsigned)(S * (N / kTile))), dim3(64 * kWaves), 0, stream,
                       f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((unsigned)(S * (N / kTile))), dim3(64 * kWaves), 0, stream, f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdLaunch& L, hipStream_t stream) {
  return L.head_dim == 64 ? launch_d<64>(L, stream) : launch_d<32>(L, stream);
}

}  // namespace mosaic
