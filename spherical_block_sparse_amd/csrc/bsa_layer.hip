// The BSA encoder layer around the attention operator: input projections to
// per-head q, k, v and branch gates, and the output projection with the
// residual.
//
// Source: papernotes.org ICML2026 notes on "(Sparse) Attention to the
// Details", 关键设计: the encoder runs several BSA layers at native HEALPix
// resolution, and BSA mixes its three branches with per-token gates g_CG,
// g_FG, g_L.  The pages give neither the projections nor the gate
// parametrisation; the layer here is the plain reading:
//   [q | k | v | z] = x W_inᵀ,  g = sigmoid(z)  (one gate per head and branch)
//   y = x + merge_heads(BSA(q, k, v, g)) W_outᵀ
// with bf16 activations between the steps (q, k, v, the merged attention
// output and y are rounded to bf16 once, round-to-nearest-even).
//
// Both projections are GEMMs D[m][n] = sum_k A[m][k] B[n][k] (A: tokens x K,
// B: features x K, both with K contiguous) with v_mfma_f32_16x16x32_bf16:
//   * bf16 operands, 256 or more output features (the input projection, and
//     the output projection from the attention output that the fine
//     kernel's merged mode writes in bf16 with the heads side by side): a
//     workgroup owns a 256-token x 256-feature tile, eight waves in 4 x 2,
//     each 64 tokens x 128 features (128 accumulator registers); K streams
//     through two 64 KB LDS stages by direct global->LDS loads into
//     XOR-swizzled rows; fewer than 256 features use 256 x 128 tiles with
//     three stages;
//   * the stage entry point's float32 [b][H][N][d] attention output is
//     instead loaded into registers one chunk ahead, rounded to bf16 and
//     written to LDS, in 128 x 128 tiles of four waves;
//   * the MFMA computes the transposed tile (features x tokens), so each
//     lane ends with four consecutive features of one token; the epilogue
//     stages a wave's 64 x 64 results through LDS and stores whole 128-byte
//     rows (the head split of q, k, v, or x + the projection); the sigmoid
//     gate logits are stored from registers;
//   * workgroups are renumbered so each XCD runs a contiguous run of tiles:
//     the feature tiles of one token tile then share its rows in one L2.
#include "bsa_common.h"

#include <math.h>

namespace mosaic {
namespace {

constexpr int kGT = 128;   // tokens and features per workgroup tile
constexpr int kGK = 64;    // K per staged chunk
constexpr int kGWaves = 4;

__device__ const uint4 kZero16L = {0u, 0u, 0u, 0u};

// 16-byte chunk swizzle of a 64-element (128-byte) row: the 8 lanes that one
// LDS cycle serves read 8 consecutive rows at the same logical chunk, which
// land on 8 different bank groups
__device__ __forceinline__ int gswz(int row) { return row & 7; }

// operand of rows 16*rt .. +15 of a staged [128][64] tile (two swizzled
// [64][64] halves): lane lr + 16*lg holds row 16*rt + lr, k = 32*kk + 8*lg .. +7
__device__ __forceinline__ bf16x8 tile_operand(const uint16_t* buf, int rt, int kk) {
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int row = 16 * rt + lr;
  return *reinterpret_cast<const bf16x8*>(buf + row * kGK + 8 * ((4 * kk + lg) ^ gswz(row)));
}

// direct loads of rows r0 .. r0+NROWS-1, k0 .. k0+63 of a [rows][K] bf16
// matrix into a staged tile; rows >= `rows` read as zeros.  Each 1 KB load
// covers 8 rows of 128 bytes; wave w of WAVES issues loads w, w+WAVES, ...
template <int NROWS = kGT, int WAVES = kGWaves>
__device__ __forceinline__ void stage_bf16(uint16_t* buf, const uint16_t* base, long long r0, long long rows,
                                           int K, int k0, int w) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int i = 0; i < NROWS / 8 / WAVES; ++i) {
    const int grp = w + WAVES * i;
    const int row = 8 * grp + lane / 8;
    const int lc = (lane % 8) ^ gswz(row);
    const long long r = r0 + row;
    const void* src = r < rows ? (const void*)(base + r * K + k0 + 8 * lc) : (const void*)&kZero16L;
    dma_global(buf + grp * 512, src);
  }
}

struct GemmArgs {
  const uint16_t* a;       // bf16 [M][K] (input projection: x)
  const float* a_heads;    // float32 [b][H][N][d] (output projection: the attention output)
  const uint16_t* b;       // bf16 [F][K] weights
  long long M;             // tokens b*N
  int F;                   // output features
  int K;
  int n_tok, heads, head_dim;
  // input projection outputs
  uint16_t* q;             // bf16 [b][H][N][d]
  uint16_t* k;
  uint16_t* v;
  float* gates;            // float32 [b][H][N][3]
  // output projection
  const uint16_t* x;       // bf16 [M][F] residual
  uint16_t* y;             // bf16 [M][F]
  int m_tiles, f_tiles;
};

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Epilogue of a wave's 64 x 64 tile: lane holds features
// f = f0 + 64*wf + 16*ft + 4*lg + i of token m = m0 + 64*wm + 16*mt + lr;
// the tile's first token is batch element bi0, position t0.
template <bool OUT>
__device__ __forceinline__ void epilogue(const GemmArgs p, const floatx4 (&acc)[4][4], long long m0, int f0,
                                         long long bi0, int t0, int wm, int wf) {
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  // the wave's 16-feature groups lie inside one head (head_dim is 32 or 64):
  // which of q, k, v, the head and the first dimension of group ft
  const int hd = p.heads * p.head_dim;
  int g_which[4], g_head[4], g_j0[4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    const int fg = __builtin_amdgcn_readfirstlane(f0 + 64 * wf + 16 * ft);
    g_which[ft] = fg / hd;
    g_head[ft] = (fg % hd) / p.head_dim;
    g_j0[ft] = fg % p.head_dim;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = 64 * wm + 16 * mt + lr;
    const long long m = m0 + row;
    if (m >= p.M) continue;
    int t = t0 + row;
    long long bi = bi0;
    while (t >= p.n_tok) {   // a tile spans at most three batch elements (N >= 192)
      t -= p.n_tok;
      bi += 1;
    }
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) {
      const int f = f0 + 64 * wf + 16 * ft + 4 * lg;
      if (f >= p.F) continue;
      const floatx4 r = acc[ft][mt];
      if constexpr (OUT) {
        const ushort4 xr = *reinterpret_cast<const ushort4*>(p.x + m * p.F + f);
        ushort4 o;
        o.x = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr.x << 16) + r[0]);
        o.y = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr.y << 16) + r[1]);
        o.z = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr.z << 16) + r[2]);
        o.w = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr.w << 16) + r[3]);
        *reinterpret_cast<ushort4*>(p.y + m * p.F + f) = o;
      } else {
        if (g_which[ft] < 3) {   // four features of one head of one of q, k, v
          const int which = g_which[ft], h = g_head[ft], j = g_j0[ft] + 4 * lg;
          uint16_t* dst = which == 0 ? p.q : (which == 1 ? p.k : p.v);
          ushort4 o;
          o.x = bf16_rne(r[0]); o.y = bf16_rne(r[1]); o.z = bf16_rne(r[2]); o.w = bf16_rne(r[3]);
          *reinterpret_cast<ushort4*>(dst + ((bi * p.heads + h) * (long long)p.n_tok + t) * p.head_dim + j) = o;
        } else {            // gate logits: feature 3*hd + 3*h + branch
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int gi = f + i - 3 * hd;
            if (gi >= 3 * p.heads) break;
            const int h = gi / 3, br = gi % 3;
            p.gates[((bi * p.heads + h) * (long long)p.n_tok + t) * 3 + br] =
                __builtin_amdgcn_rcpf(1.f + __expf(-r[i]));
          }
        }
      }
    }
  }
}

// Epilogue through LDS: the wave's 64 x 64 float32 tile goes to its own LDS
// region (rows padded by 16 bytes against bank conflicts), then is read back
// a token row at a time, so every global store writes whole 128-byte runs
// (a head's 64 dims of q, k or v, or 64 channels of y) instead of 32-byte
// pieces of four different lines.  Gate-logit features keep the direct path.
template <bool OUT>
__device__ __forceinline__ void epilogue_staged(const GemmArgs p, const floatx4 (&acc)[4][4], long long m0, int f0,
                                                long long bi0, int t0, int wm, int wf, float* lds) {
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int fw = f0 + 64 * wf;   // the wave's first feature, uniform
  const int hd = p.heads * p.head_dim;
  if (fw >= p.F) return;
  if (!OUT && fw >= 3 * hd) {   // gate logits
    epilogue<false>(p, acc, m0, f0, bi0, t0, wm, wf);
    return;
  }
  constexpr int RS = 64 + 4;   // floats per staged row
  const int cl = lane % 16;             // 16-byte piece (4 features) of the row
  const int fl = fw + 4 * cl;           // this lane's first feature
  const bool f_ok = fl < p.F;
  const int r0 = lane / 16;             // first row of this lane; rows r0, r0 + 4, ...
  const long long mw = m0 + 64 * wm;    // the wave's first token
  const long long rows_left = p.M - mw; // rows of the wave that exist
  // OUT: the residual rows this lane adds, all loaded before anything is
  // stored (x and y may alias as far as the compiler knows, so loads issued
  // between the stores would each wait for the one before)
  ushort4 xr[16];
  if constexpr (OUT) {
    const uint16_t* xp = p.x + (mw + r0) * p.F + fl;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      xr[i] = 4 * i + r0 < rows_left && f_ok ? *reinterpret_cast<const ushort4*>(xp + 4LL * i * p.F)
                                             : make_ushort4(0, 0, 0, 0);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
      *reinterpret_cast<floatx4*>(lds + (16 * mt + lr) * RS + 16 * ft + 4 * lg) = acc[ft][mt];
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's own LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // the wave's first token: batch element bw, position tw (a tile spans at
  // most two batch elements per wave: 64 rows, N >= 192)
  long long bw = bi0;
  int tw = t0 + 64 * wm;
  if (tw >= p.n_tok) {
    tw -= p.n_tok;
    bw += 1;
  }
  // per-row global pointers: rows before the batch boundary, and after it
  uint16_t* row0 = nullptr;
  uint16_t* row1 = nullptr;
  int step = 0;
  if constexpr (OUT) {
    row0 = p.y + mw * p.F + fl;
    step = p.F;
  } else {
    const int which = fw / hd, h = (fl % hd) / p.head_dim, j = fl % p.head_dim;
    uint16_t* dst = which == 0 ? p.q : (which == 1 ? p.k : p.v);
    row0 = dst + ((bw * p.heads + h) * (long long)p.n_tok + tw) * p.head_dim + j;
    row1 = dst + ((bw + 1) * p.heads + h) * (long long)p.n_tok * p.head_dim + j;
    step = p.head_dim;
  }
  const int split = p.n_tok - tw;       // rows from here on belong to batch element bw + 1
  if (OUT || split >= 64) {             // one batch element: pointers advance by 4 rows
    uint16_t* yp = row0 + (long long)r0 * step;
    const long long adv = 4LL * step;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + r0;
      if (row < rows_left && f_ok) {
        const floatx4 r = *reinterpret_cast<const floatx4*>(lds + row * RS + 4 * cl);
        ushort4 o;
        if constexpr (OUT) {
          o.x = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr[i].x << 16) + r[0]);
          o.y = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr[i].y << 16) + r[1]);
          o.z = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr[i].z << 16) + r[2]);
          o.w = bf16_rne(__builtin_bit_cast(float, (uint32_t)xr[i].w << 16) + r[3]);
        } else {
          o.x = bf16_rne(r[0]); o.y = bf16_rne(r[1]); o.z = bf16_rne(r[2]); o.w = bf16_rne(r[3]);
        }
        *reinterpret_cast<ushort4*>(yp) = o;
      }
      yp += adv;
    }
    return;
  }
  // a tile that crosses into the next batch element (q, k, v only)
  for (int i = 0; i < 16; ++i) {
    const int row = 4 * i + r0;
    if (row >= rows_left || !f_ok) continue;
    const floatx4 r = *reinterpret_cast<const floatx4*>(lds + row * RS + 4 * cl);
    uint16_t* d = row < split ? row0 + (long long)row * step : row1 + (long long)(row - split) * step;
    ushort4 o;
    o.x = bf16_rne(r[0]); o.y = bf16_rne(r[1]); o.z = bf16_rne(r[2]); o.w = bf16_rne(r[3]);
    *reinterpret_cast<ushort4*>(d) = o;
  }
}

// The output projection (residual epilogue) from the float32 [b][H][N][d]
// attention output of the stage entry point: 128 x 128 tiles on four waves,
// A loaded into registers one chunk ahead and rounded to bf16 into LDS.
template <bool OUT>
__global__ __launch_bounds__(64 * kGWaves) void layer_gemm_a32_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGT * kGK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGT * kGK];
  const long long tiles = (long long)p.m_tiles * p.f_tiles;
  long long logical;
  {
    const long long b = blockIdx.x, q8 = tiles / 8, r8 = tiles % 8, xcd = b % 8, kq = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + kq : r8 * (q8 + 1) + (xcd - r8) * q8 + kq;
  }
  const long long m0 = (logical / p.f_tiles) * kGT;
  const int f0 = (int)(logical % p.f_tiles) * kGT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, lr = lane % 16, lg = lane / 16;
  const int wm = w & 1, wf = w >> 1;   // the wave's 64-token and 64-feature quarter
  const int nk = p.K / kGK;
  // the tile's first token is batch element bi0, position t0 (one division
  // per workgroup); a tile of 128 tokens spans at most two batch elements
  // (N >= 192)
  const long long bi0 = m0 / p.n_tok;
  const int t0 = (int)(m0 - bi0 * p.n_tok);

  // OUT: the float32 attention output of chunk c, rows m0 .. m0+127: thread
  // x handles row x/2, 32 of its 64 k values (8 float4), k = 32*(x%2) + 4*i
  const int ar = threadIdx.x / 2, ah = threadIdx.x % 2;
  float4 areg[8];
  const bool a_ok = m0 + ar < p.M;
  const long long a_row = (t0 + ar < p.n_tok) ? bi0 * p.heads * (long long)p.n_tok + t0 + ar
                                               : (bi0 + 1) * p.heads * (long long)p.n_tok + t0 + ar - p.n_tok;
  auto load_a32 = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = c * kGK + 32 * ah + 4 * i;          // feature h*d + j of the merged heads
      const int h = kk / p.head_dim, j = kk % p.head_dim;
      areg[i] = a_ok ? *reinterpret_cast<const float4*>(
                           p.a_heads + ((a_row + (long long)h * p.n_tok) * p.head_dim + j))
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_a32 = [&](uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {   // two float4 = one 16-byte chunk of 8 bf16
      const int kc = 32 * ah + 4 * i;  // k within the chunk, a multiple of 8
      ushort4 lo, hi;
      lo.x = bf16_rne(areg[i].x); lo.y = bf16_rne(areg[i].y); lo.z = bf16_rne(areg[i].z); lo.w = bf16_rne(areg[i].w);
      hi.x = bf16_rne(areg[i + 1].x); hi.y = bf16_rne(areg[i + 1].y);
      hi.z = bf16_rne(areg[i + 1].z); hi.w = bf16_rne(areg[i + 1].w);
      uint16_t* dst = buf + ar * kGK + 8 * ((kc / 8) ^ gswz(ar));
      *reinterpret_cast<ushort4*>(dst) = lo;
      *reinterpret_cast<ushort4*>(dst + 4) = hi;
    }
  };
  auto stage = [&](int c, int s) __attribute__((always_inline)) {
    stage_bf16(Bs[s], p.b, f0, p.F, p.K, c * kGK, w);
  };

  floatx4 acc[4][4];   // [feature tile][token tile]: features 16*ft + 4*lg + i of token 16*mt + lr
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[ft][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  load_a32(0);
  store_a32(As[0]);
  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads have landed
  __syncthreads();
  for (int c = 0; c < nk; ++c) {
    const int s = c & 1;
    if (c + 1 < nk) {
      stage(c + 1, s ^ 1);
      load_a32(c + 1);
    }
    const uint16_t* a_t = As[s] + wm * 64 * kGK;
    const uint16_t* b_t = Bs[s] + wf * 64 * kGK;
#pragma unroll
    for (int kk = 0; kk < kGK / 32; ++kk) {
      bf16x8 bo[4], ao[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bo[t] = tile_operand(b_t, t, kk);
        ao[t] = tile_operand(a_t, t, kk);
      }
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[ft][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo[ft], ao[mt], acc[ft][mt], 0, 0, 0);
    }
    // buffer s^1 was last read in chunk c-1, before the barrier that ended it
    if (c + 1 < nk) store_a32(As[s ^ 1]);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  epilogue<OUT>(p, acc, m0, f0, bi0, t0, wm, wf);
}

// Both operands bf16, fewer than 256 output features: 256-token x
// 128-feature tiles, 8 waves in 4 x 2 (each 64 x 64, two per SIMD, one
// workgroup per CU), three LDS stages (144 KB): chunk c+2 loads while c is
// computed, so two chunks of loads are in flight per CU.
constexpr int kBT = 256;
constexpr int kBWaves = 8;

template <bool OUT>
__global__ __launch_bounds__(64 * kBWaves) void layer_gemm_big_kernel(GemmArgs p) {
  // three A stages (256 x 64) then three B stages (128 x 64), one array so
  // that the epilogue can reuse all of it
  __shared__ __attribute__((aligned(16))) uint16_t smem[3 * kBT * kGK + 3 * kGT * kGK];
  auto As = [&](int st) __attribute__((always_inline)) { return smem + st * kBT * kGK; };
  auto Bs = [&](int st) __attribute__((always_inline)) { return smem + 3 * kBT * kGK + st * kGT * kGK; };
  const long long tiles = (long long)p.m_tiles * p.f_tiles;
  long long logical;
  {
    const long long b = blockIdx.x, q8 = tiles / 8, r8 = tiles % 8, xcd = b % 8, kq = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + kq : r8 * (q8 + 1) + (xcd - r8) * q8 + kq;
  }
  const long long m0 = (logical / p.f_tiles) * kBT;
  const int f0 = (int)(logical % p.f_tiles) * kGT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w & 3, wf = w >> 2;   // the wave's 64-token and 64-feature part
  const int nk = p.K / kGK;
  const long long bi0 = m0 / p.n_tok;
  const int t0 = (int)(m0 - bi0 * p.n_tok);
  // loads per wave and chunk: (256 + 128) rows / 8 rows per load / 8 waves
  constexpr int kLoadsA = kBT / 8 / kBWaves, kLoadsB = kGT / 8 / kBWaves;
  constexpr int kLoads = kLoadsA + kLoadsB;
  // per-lane source pointers of the wave's loads, formed once: load i covers
  // rows 8*(w + 8i) .. +7, the lane one 16-byte piece of one row.  Rows past
  // the matrix are clamped to its last row: they only feed accumulator rows
  // or columns that the epilogue never stores.  A chunk then only adds its
  // k offset.
  const int lane = threadIdx.x % kWave;
  const uint16_t* srcA[kLoadsA];
  const uint16_t* srcB[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int row = 8 * (w + kBWaves * i) + lane / 8;
    const long long r = m0 + row < p.M ? m0 + row : p.M - 1;
    srcA[i] = p.a + r * p.K + 8 * ((lane % 8) ^ gswz(row));
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int row = 8 * (w + kBWaves * i) + lane / 8;
    const long long r = f0 + row < p.F ? f0 + row : p.F - 1;
    srcB[i] = p.b + r * p.K + 8 * ((lane % 8) ^ gswz(row));
  }
  const int lds_wave = lds_addr(smem) + w * 1024;   // the wave's first 1 KB slot
  auto stage = [&](int c, int s) __attribute__((always_inline)) {
    const int k0 = c * kGK;
    const int a_base = __builtin_amdgcn_readfirstlane(lds_wave + s * (kBT * kGK * 2));
    const int b_base = __builtin_amdgcn_readfirstlane(lds_wave + 3 * (kBT * kGK * 2) + s * (kGT * kGK * 2));
    static_for<0, kLoadsA>([&](auto i) __attribute__((always_inline)) {
      dma_global_at<decltype(i)::value * kBWaves * 1024>(a_base, srcA[decltype(i)::value] + k0);
    });
    static_for<0, kLoadsB>([&](auto i) __attribute__((always_inline)) {
      dma_global_at<decltype(i)::value * kBWaves * 1024>(b_base, srcB[decltype(i)::value] + k0);
    });
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[ft][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  stage(0, 0);
  if (nk > 1) {
    stage(1, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);   // chunk 0 has landed (loads complete in order)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  __syncthreads();
  int s = 0;
  for (int c = 0; c < nk; ++c) {
    // buffer (c+2)%3 was last read in chunk c-1, before the barrier that ended it
    if (c + 2 < nk) stage(c + 2, s == 0 ? 2 : s - 1);
    const uint16_t* a_t = As(s) + wm * 64 * kGK;
    const uint16_t* b_t = Bs(s) + wf * 64 * kGK;
#pragma unroll
    for (int kk = 0; kk < kGK / 32; ++kk) {
      bf16x8 bo[4], ao[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bo[t] = tile_operand(b_t, t, kk);
        ao[t] = tile_operand(a_t, t, kk);
      }
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[ft][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo[ft], ao[mt], acc[ft][mt], 0, 0, 0);
    }
    if (c + 2 < nk)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);   // chunk c+1 has landed, c+2 may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    s = s == 2 ? 0 : s + 1;
  }
  // the staging buffers are free (every wave passed the last barrier): each
  // wave takes a 64 x 68 float region of them (8 x 17 KB of the 144 KB)
  epilogue_staged<OUT>(p, acc, m0, f0, bi0, t0, wm, wf, reinterpret_cast<float*>(smem) + w * 64 * (64 + 4));
}

// 256 x 256 tiles: twice the FLOPs per staged byte of the 256 x 128 kernel.
// 8 waves in 4 x 2, each 64 tokens x 128 features (32 MFMA tiles); two LDS
// stages of 64 KB, the next chunk loading while one is computed (the same
// 2048 clocks of MFMA work in flight ahead of the loads as three stages of
// the narrower tile); the epilogue stages each 64-feature half of a wave's
// tile through LDS.
constexpr int kWT = 256;
constexpr int kWRS = 64 + 4;   // floats per staged epilogue row
constexpr int kWSmem = (2 * 2 * kWT * kGK) > (kBWaves * 64 * kWRS * 2) ? (2 * 2 * kWT * kGK) : (kBWaves * 64 * kWRS * 2);

template <bool OUT>
__global__ __launch_bounds__(64 * kBWaves) void layer_gemm_wide_kernel(GemmArgs p) {
  // stage s: A (256 x 64) at s * 2*kWT*kGK, then B (256 x 64); the epilogue
  // reuses the whole array (uint16 units)
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWSmem];
  auto As = [&](int st) __attribute__((always_inline)) { return smem + st * 2 * kWT * kGK; };
  auto Bs = [&](int st) __attribute__((always_inline)) { return smem + st * 2 * kWT * kGK + kWT * kGK; };
  const long long tiles = (long long)p.m_tiles * p.f_tiles;
  long long logical;
  {
    const long long b = blockIdx.x, q8 = tiles / 8, r8 = tiles % 8, xcd = b % 8, kq = b / 8;
    logical = xcd < r8 ? xcd * (q8 + 1) + kq : r8 * (q8 + 1) + (xcd - r8) * q8 + kq;
  }
  const long long m0 = (logical / p.f_tiles) * kWT;
  const int f0 = (int)(logical % p.f_tiles) * kWT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w & 3, wf = w >> 2;   // the wave's 64-token and 128-feature part
  const int nk = p.K / kGK;
  const long long bi0 = m0 / p.n_tok;
  const int t0 = (int)(m0 - bi0 * p.n_tok);
  constexpr int kLoadsA = kWT / 8 / kBWaves, kLoadsB = kWT / 8 / kBWaves;   // 4 + 4 per wave and chunk
  constexpr int kLoads = kLoadsA + kLoadsB;
  // per-lane source pointers, formed once (rows past the matrix clamped to
  // its last row: they only feed results the epilogue never stores)
  const int lane = threadIdx.x % kWave;
  const uint16_t* srcA[kLoadsA];
  const uint16_t* srcB[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int row = 8 * (w + kBWaves * i) + lane / 8;
    const long long r = m0 + row < p.M ? m0 + row : p.M - 1;
    srcA[i] = p.a + r * p.K + 8 * ((lane % 8) ^ gswz(row));
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int row = 8 * (w + kBWaves * i) + lane / 8;
    const long long r = f0 + row < p.F ? f0 + row : p.F - 1;
    srcB[i] = p.b + r * p.K + 8 * ((lane % 8) ^ gswz(row));
  }
  const int lds_wave = lds_addr(smem) + w * 1024;   // the wave's first 1 KB slot
  auto stage = [&](int c, int s) __attribute__((always_inline)) {
    const int k0 = c * kGK;
    const int a_base = __builtin_amdgcn_readfirstlane(lds_wave + s * (2 * kWT * kGK * 2));
    const int b_base = __builtin_amdgcn_readfirstlane(lds_wave + s * (2 * kWT * kGK * 2) + kWT * kGK * 2);
    static_for<0, kLoadsA>([&](auto i) __attribute__((always_inline)) {
      dma_global_at<decltype(i)::value * kBWaves * 1024>(a_base, srcA[decltype(i)::value] + k0);
    });
    static_for<0, kLoadsB>([&](auto i) __attribute__((always_inline)) {
      dma_global_at<decltype(i)::value * kBWaves * 1024>(b_base, srcB[decltype(i)::value] + k0);
    });
  };
  floatx4 acc[8][4];
#pragma unroll
  for (int ft = 0; ft < 8; ++ft)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[ft][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int c = 0; c < nk; ++c) {
    const int s = c & 1;
    // stage s^1 was last read in chunk c-1, before the barrier that ended it
    if (c + 1 < nk) stage(c + 1, s ^ 1);
    const uint16_t* a_t = As(s) + wm * 64 * kGK;
    const uint16_t* b_t = Bs(s) + wf * 128 * kGK;
#pragma unroll
    for (int kk = 0; kk < kGK / 32; ++kk) {
      bf16x8 bo[8], ao[4];
#pragma unroll
      for (int t = 0; t < 8; ++t) bo[t] = tile_operand(b_t, t, kk);
#pragma unroll
      for (int t = 0; t < 4; ++t) ao[t] = tile_operand(a_t, t, kk);
#pragma unroll
      for (int ft = 0; ft < 8; ++ft)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[ft][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bo[ft], ao[mt], acc[ft][mt], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // chunk c+1 has landed
    __syncthreads();
  }
  // the stages are free (every wave passed the last barrier): each wave takes
  // a 64 x 68 float region and writes its two 64-feature halves in turn (a
  // wave's own LDS reads and writes are processed in order)
  float* lds = reinterpret_cast<float*>(smem) + w * 64 * kWRS;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    floatx4 half[4][4];
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) half[ft][mt] = acc[4 * h + ft][mt];
    epilogue_staged<OUT>(p, half, m0, f0 + 128 * wf + 64 * h, bi0, t0, wm, 0, lds);
  }
}

hipError_t launch_gemm(GemmArgs p, bool out, bool a32, hipStream_t stream) {
  p.f_tiles = (p.F + kGT - 1) / kGT;
  if (a32) {
    p.m_tiles = (int)((p.M + kGT - 1) / kGT);
    const dim3 grid((unsigned)((long long)p.m_tiles * p.f_tiles));
    hipLaunchKernelGGL(layer_gemm_a32_kernel<true>, grid, dim3(64 * kGWaves), 0, stream, p);
    return hipGetLastError();
  }
  if (p.F >= kWT) {   // 256 x 256 tiles
    p.f_tiles = (p.F + kWT - 1) / kWT;
    p.m_tiles = (int)((p.M + kWT - 1) / kWT);
    const dim3 grid((unsigned)((long long)p.m_tiles * p.f_tiles));
    if (out)
      hipLaunchKernelGGL(layer_gemm_wide_kernel<true>, grid, dim3(64 * kBWaves), 0, stream, p);
    else
      hipLaunchKernelGGL(layer_gemm_wide_kernel<false>, grid, dim3(64 * kBWaves), 0, stream, p);
    return hipGetLastError();
  }
  p.m_tiles = (int)((p.M + kBT - 1) / kBT);
  const dim3 grid((unsigned)((long long)p.m_tiles * p.f_tiles));
  if (out)
    hipLaunchKernelGGL(layer_gemm_big_kernel<true>, grid, dim3(64 * kBWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(layer_gemm_big_kernel<false>, grid, dim3(64 * kBWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_in(const uint16_t* x, const uint16_t* w_in, long long batch, int n_tok, int channels,
                           int heads, int head_dim, uint16_t* q, uint16_t* k, uint16_t* v, float* gates,
                           hipStream_t stream) {
  GemmArgs p = {};
  p.a = x;
  p.b = w_in;
  p.M = batch * n_tok;
  p.F = 3 * heads * head_dim + 3 * heads;
  p.K = channels;
  p.n_tok = n_tok;
  p.heads = heads;
  p.head_dim = head_dim;
  p.q = q;
  p.k = k;
  p.v = v;
  p.gates = gates;
  return launch_gemm(p, false, false, stream);
}

hipError_t launch_layer_out(const float* attn, const uint16_t* w_out, const uint16_t* x, long long batch,
                            int n_tok, int channels, int heads, int head_dim, uint16_t* y, hipStream_t stream) {
  GemmArgs p = {};
  p.a_heads = attn;
  p.b = w_out;
  p.M = batch * n_tok;
  p.F = channels;
  p.K = heads * head_dim;
  p.n_tok = n_tok;
  p.heads = heads;
  p.head_dim = head_dim;
  p.x = x;
  p.y = y;
  return launch_gemm(p, true, true, stream);
}

hipError_t launch_layer_out_merged(const uint16_t* attn_merged, const uint16_t* w_out, const uint16_t* x,
                                   long long batch, int n_tok, int channels, int heads, int head_dim, uint16_t* y,
                                   hipStream_t stream) {
  GemmArgs p = {};
  p.a = attn_merged;
  p.b = w_out;
  p.M = batch * n_tok;
  p.F = channels;
  p.K = heads * head_dim;
  p.n_tok = n_tok;
  p.heads = heads;
  p.head_dim = head_dim;
  p.x = x;
  p.y = y;
  return launch_gemm(p, true, false, stream);
}

}  // namespace mosaic
