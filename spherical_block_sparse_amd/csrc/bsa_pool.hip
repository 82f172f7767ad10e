// Block pooling: mean of every `block` consecutive NESTED tokens of q, k, v.
//
// Source: papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse
// Attention (block summaries q̄, k̄, v̄ by a pooling phi; the mean is the
// reading taken here) and › HEALPix + NESTED (a block is a contiguous index
// range, so it is read in one coalesced sweep).
//
// Layout: x [slices][N][D] bf16 -> xbar [slices][m][D]; q̄, k̄ in float64, v̄
// in float32.  A block is block*D*2 contiguous bytes.
//
// Mapping: D/8 lanes cover one token row (16 bytes = 8 bf16 each), so a
// 256-thread workgroup streams 256/(D/8) blocks side by side, every lane
// walking its 16-byte column slice down all rows of its block.  Each wave
// instruction touches 64/(D/8) full 128-byte (D=64) row segments; no
// cross-lane reduction is needed.  A sweep step loads 8 rows; blocks of 1 or
// 4 tokens take one row per step.  Sums are float64: exact for bf16 inputs
// (8-bit significands, at most a few thousand terms), and block = 4^k makes
// the final scaling exact.  HBM-bound: 6*D bytes read per token.
//
// With kpieces, the key workgroups also write k̄ as two bf16 pieces and each
// block's |k̄|^2, the inputs of the approximate compressed-branch logits.
//
// The key workgroups can also write each block's largest key norm
// max_t |k_t| (float32 [slices][m]).  It is not part of the method: the
// fine-attention kernel turns it into an upper bound on a query's scores
// over a set of blocks (Cauchy-Schwarz: q.k <= |q| |k|) and then needs no
// running maximum.
#include "bsa_common.h"

namespace mosaic {
namespace {

struct PoolArgs {
  const uint16_t* src[3];
  double* dst64[2];   // q̄, k̄
  float* dst32;       // v̄
  float* knorm;       // largest key norm of each block, or null
  uint16_t* kpieces;  // bf16 pieces of k̄ [slices][m][2][D], or null
  float* kbn2;        // |k̄_j|^2 of each block [slices][m] (rounded up), with kpieces
  long long total_blocks;   // slices * m
  long long wgs_per_tensor;
  int block;
  double inv_block;
};

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int TPR = D / 8;              // lanes per token row
  constexpr int BPW = 256 / TPR;          // blocks per workgroup
  const int tensor = (int)(blockIdx.x / a.wgs_per_tensor);
  const long long wg = blockIdx.x - (long long)tensor * a.wgs_per_tensor;
  const int lb = threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  const long long gb = wg * BPW + lb;
  if (gb >= a.total_blocks) return;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* p = reinterpret_cast<const u32x4*>(a.src[tensor] + (size_t)gb * a.block * D) + c;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;

  // NORM: also track the largest squared key norm.  Lane c holds channels
  // 8c .. 8c+7 of a row, so a row's |k|^2 is a sum over the row's TPR
  // lanes: each lane forms its 8-channel partials of 8 rows, and a
  // butterfly over the TPR lanes (each step hands half of the rows to the
  // partner and adds the partner's share of the other half) leaves every
  // lane with whole sums of 8/TPR of them.
  auto sweep = [&](auto NORM) __attribute__((always_inline)) {
    float nmax = 0.f;
    for (int r0 = 0; r0 < a.block; r0 += 8) {
      u32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = __builtin_nontemporal_load(p + (size_t)(r0 + u) * TPR);
      float ss[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t x[4] = {w[u][0], w[u][1], w[u][2], w[u][3]};
        ss[u] = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float lo = __uint_as_float(x[h] << 16), hi = __uint_as_float(x[h] & 0xffff0000u);
          acc[2 * h] += (double)lo;
          acc[2 * h + 1] += (double)hi;
          if constexpr (decltype(NORM)::value) ss[u] = fmaf(hi, hi, fmaf(lo, lo, ss[u]));
        }
      }
      if constexpr (decltype(NORM)::value) {
        static_for<0, 3>([&](auto st) __attribute__((always_inline)) {
          constexpr int off = TPR >> (1 + decltype(st)::value), half = 4 >> decltype(st)::value;
          if constexpr (off >= 1) {
            const bool upper = (c & off) != 0;
#pragma unroll
            for (int i = 0; i < half; ++i) {
              const float send = upper ? ss[i] : ss[i + half];
              const float keep = upper ? ss[i + half] : ss[i];
              ss[i] = keep + __shfl_xor(send, off);
            }
          }
        });
        constexpr int left = 8 / TPR;   // whole row sums now held by each lane
#pragma unroll
        for (int i = 0; i < left; ++i) nmax = fmaxf(nmax, ss[i]);
      }
    }
    if constexpr (decltype(NORM)::value) {
      // the TPR lanes of a block are consecutive and TPR-aligned
#pragma unroll
      for (int off = 1; off < TPR; off *= 2) nmax = fmaxf(nmax, __shfl_xor(nmax, off));
      if (c == 0) a.knorm[gb] = sqrtf(nmax);
    }
  };
  // blocks of 1 or 4 tokens (fewer than the 8 rows a sweep step loads): one
  // row per step, each row's |k|^2 summed over its TPR lanes
  auto sweep_small = [&](auto NORM) __attribute__((always_inline)) {
    float nmax = 0.f;
    for (int r = 0; r < a.block; ++r) {
      const u32x4 w = __builtin_nontemporal_load(p + (size_t)r * TPR);
      const uint32_t x[4] = {w[0], w[1], w[2], w[3]};
      float ss = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float lo = __uint_as_float(x[h] << 16), hi = __uint_as_float(x[h] & 0xffff0000u);
        acc[2 * h] += (double)lo;
        acc[2 * h + 1] += (double)hi;
        if constexpr (decltype(NORM)::value) ss = fmaf(hi, hi, fmaf(lo, lo, ss));
      }
      if constexpr (decltype(NORM)::value) {
#pragma unroll
        for (int off = 1; off < TPR; off *= 2) ss += __shfl_xor(ss, off);
        nmax = fmaxf(nmax, ss);
      }
    }
    if constexpr (decltype(NORM)::value) {
      if (c == 0) a.knorm[gb] = sqrtf(nmax);
    }
  };
  if (a.block < 8) {
    if (tensor == 1 && a.knorm)
      sweep_small(std::true_type{});
    else
      sweep_small(std::false_type{});
  } else if (tensor == 1 && a.knorm) {
    sweep(std::true_type{});
  } else {
    sweep(std::false_type{});
  }

  const size_t o = (size_t)gb * D + c * 8;
  if (tensor < 2) {
    double* dst = a.dst64[tensor] + o;
    double2* d2 = reinterpret_cast<double2*>(dst);
#pragma unroll
    for (int j = 0; j < 4; ++j) d2[j] = make_double2(acc[2 * j] * a.inv_block, acc[2 * j + 1] * a.inv_block);
    if (tensor == 1 && a.kpieces) {
      // k̄ = k1 + k2 + r with k1 = bf16(k̄), k2 = bf16(k̄ - k1) (through float32:
      // |r| <= (2^-16 + 2^-24)|k̄|), natural channel order, and |k̄|^2 of the
      // block (the approximate selection's error bound)
      uint4 p1, p2;
      uint32_t* w1 = reinterpret_cast<uint32_t*>(&p1);
      uint32_t* w2 = reinterpret_cast<uint32_t*>(&p2);
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t b1[2], b2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const double x = acc[2 * j + h] * a.inv_block;
          const float xf = static_cast<float>(x);
          const __bf16 k1 = static_cast<__bf16>(xf);
          const __bf16 k2 = static_cast<__bf16>(xf - static_cast<float>(k1));
          b1[h] = __builtin_bit_cast(uint16_t, k1);
          b2[h] = __builtin_bit_cast(uint16_t, k2);
          ss = fma(x, x, ss);
        }
        w1[j] = b1[0] | (b1[1] << 16);
        w2[j] = b2[0] | (b2[1] << 16);
      }
      uint16_t* prow = a.kpieces + (size_t)gb * 2 * D + c * 8;
      *reinterpret_cast<uint4*>(prow) = p1;
      *reinterpret_cast<uint4*>(prow + D) = p2;
#pragma unroll
      for (int off = 1; off < TPR; off *= 2) ss += __shfl_xor(ss, off);
      if (c == 0) a.kbn2[gb] = static_cast<float>(ss * (1.0 + 1e-6));
    }
  } else {
    float4* d4 = reinterpret_cast<float4*>(a.dst32 + o);
    d4[0] = make_float4((float)(acc[0] * a.inv_block), (float)(acc[1] * a.inv_block),
                        (float)(acc[2] * a.inv_block), (float)(acc[3] * a.inv_block));
    d4[1] = make_float4((float)(acc[4] * a.inv_block), (float)(acc[5] * a.inv_block),
                        (float)(acc[6] * a.inv_block), (float)(acc[7] * a.inv_block));
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* qbar,
                       double* kbar, float* vbar, long long slices, int n_tok, int head_dim,
                       int block, hipStream_t stream, float* knorm, uint16_t* kpieces, float* kbn2) {
  PoolArgs a;
  a.kpieces = kpieces;
  a.kbn2 = kbn2;
  a.src[0] = q;
  a.src[1] = k;
  a.src[2] = v;
  a.dst64[0] = qbar;
  a.dst64[1] = kbar;
  a.dst32 = vbar;
  a.knorm = knorm;
  a.total_blocks = slices * (long long)(n_tok / block);
  a.block = block;
  a.inv_block = 1.0 / (double)block;
  const int bpw = 256 / (head_dim / 8);
  a.wgs_per_tensor = (a.total_blocks + bpw - 1) / bpw;
  dim3 grid((unsigned)(3 * a.wgs_per_tensor));
  if (head_dim == 64)
    hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pool_kernel<32>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mosaic
