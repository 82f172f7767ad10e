// Host-side launch functions of the BSA kernels, called by the C-ABI entry
// points (mosaic_bsa_api.cpp).  Plain C++ declarations over the HIP runtime
// API: this header holds no device code, so the validation layer can also be
// built by a host compiler alone (the sanitizer build of the ABI tests).
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stddef.h>
#include <stdint.h>

namespace mosaic {

// knorm non-null: also write the largest key norm max_t |k_t| of each block, float32 [slices][m].
// kpieces, kbn2 non-null (both): also write k̄ as bf16 pieces k1 = bf16(k̄), k2 = bf16(k̄ - k1),
// [slices][m][2][head_dim] (natural channel order, k1 first), and |k̄_j|^2 per block (float32,
// rounded up), [slices][m].
hipError_t launch_pool(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* qbar,
                       double* kbar, float* vbar, long long slices, int n_tok, int head_dim,
                       int block, hipStream_t stream, float* knorm = nullptr, uint16_t* kpieces = nullptr,
                       float* kbn2 = nullptr);

// kpieces, kbn2 non-null (the pool's): topn <= 16 ranks on approximate logits from the pieces and
// certifies every row (float64 rescoring of the band at its n-th value; a row it cannot certify is
// settled by an exact float64 radix selection).  Without them, or for larger topn, the logits are
// float64 throughout.
hipError_t launch_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                  float* o_cg, int32_t* sel, long long slices, int m, int head_dim,
                                  int topn, hipStream_t stream, const uint16_t* kpieces = nullptr,
                                  const float* kbn2 = nullptr);

// knorm non-null (the pool's largest key norm per block): waves whose scores
// it bounds tightly enough skip the running maximum of the online softmax.
// save_o / save_lse non-null: also write each query's normalised selected and
// local branch outputs (float32 [S][N][2][D]) and their log2-sum-exp
// ([S][N][2]).  out_merged non-null (with `heads`, S = batch*heads): write
// out in bf16 as [batch][N][heads][D] there instead of `out`.
hipError_t launch_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gates,
                       const float* o_cg, const int32_t* sel, float* out, long long slices,
                       int n_tok, int head_dim, int block, int topn, int window,
                       hipStream_t stream, const float* knorm = nullptr, float* save_o = nullptr,
                       float* save_lse = nullptr, uint16_t* out_merged = nullptr, int heads = 1,
                       const float* selmax = nullptr);

// whether launch_fine runs the tiled kernel (the one that reads selmax)
bool fine_tiled(int n_tok, int block, int topn);

// selmax[r] = max over row r's topn selected blocks of knorm (indices clamped
// into [0, m)), r < slices * m: the selected branch's score bound per query block
hipError_t launch_sel_bound(const int32_t* sel, const float* knorm, float* sel_bound, long long slices, int m,
                            int topn, hipStream_t stream);

// Everything the backward launches read and write (device pointers; the
// workspace buffers are carved by the C-ABI entry point).
struct BwdLaunch {
  const uint16_t* q;        // bf16 [S][N][d]
  const uint16_t* k;
  const uint16_t* v;
  const float* gates;       // [S][N][3]
  const int32_t* sel;       // [S][m][topn] from the forward
  const float* dout;        // [S][N][d]
  float* dq;                // outputs, fp32 [S][N][d]
  float* dk;
  float* dv;
  float* dgates;            // [S][N][3]
  int head_dim;
  long long slices;
  int n_tok, block, topn, window;
  const double* qbar;       // pooled means [S][m][d] (recomputed, or the training forward's)
  const double* kbar;
  const float* vbar;
  const float* o_cg;        // compressed output [S][m][d] (likewise)
  const float* save_o;      // training forward's o_FG, o_L [S][N][2][d], or null: recompute
  const float* save_lse;    // their log2-sum-exp [S][N][2]
  uint16_t* dob;            // workspace: bf16 dO [S][N][d] with the sign of g_FG (selected branch)
  uint16_t* dob_loc;        // the same with the sign of g_L (local branch)
  float* docg;              // [S][m][d] and its bf16 copy
  uint16_t* docg_b;
  uint16_t* qbar_b;         // bf16 pooled rows [S][m][d]
  uint16_t* kbar_b;
  uint16_t* vbar_b;
  float* stats;             // [2][S][3][N] planes lse, D, g
  float* stats_cg;          // [2][S][3][m]
  float* dqbar;             // [S][m][d]
  float* dkbar;
  float* dvbar;
  int32_t* inv_off;         // [S][m+1]
  int32_t* inv_tmp;         // [S][m*topn] unsorted inverted lists
  int32_t* inv_list;        // [S][m*topn]
};

// Encoder layer projections (bsa_layer.hip).  Input: x [batch*N][channels]
// bf16 times w_in [3*H*d + 3*H][channels] bf16 -> q, k, v bf16 [batch][H][N][d]
// and gates = sigmoid(logits) float32 [batch][H][N][3].  Output:
// y = x + merge(attn) w_outᵀ with attn float32 [batch][H][N][d] and w_out
// [channels][H*d] bf16, y bf16 [batch*N][channels].  channels and H*d are
// multiples of 64.
hipError_t launch_layer_in(const uint16_t* x, const uint16_t* w_in, long long batch, int n_tok, int channels,
                           int heads, int head_dim, uint16_t* q, uint16_t* k, uint16_t* v, float* gates,
                           hipStream_t stream);
hipError_t launch_layer_out(const float* attn, const uint16_t* w_out, const uint16_t* x, long long batch,
                            int n_tok, int channels, int heads, int head_dim, uint16_t* y, hipStream_t stream);
// the same from the attention output already merged and in bf16, [batch*N][H*d]
hipError_t launch_layer_out_merged(const uint16_t* attn_merged, const uint16_t* w_out, const uint16_t* x,
                                   long long batch, int n_tok, int channels, int heads, int head_dim, uint16_t* y,
                                   hipStream_t stream);

// HEALPix NESTED coarsening (healpix_coarsen.hip): y [batch][N/4^levels][C]
// float32 = mean of each run of 4^levels rows of x [batch][N][C] bf16;
// C a multiple of 8.
hipError_t launch_coarsen(const uint16_t* x, float* y, long long batch, int n_tok, int channels, int levels,
                          hipStream_t stream);

// Lat-lon -> HEALPix cross-attention interpolation (healpix_interp.hip):
// k [S][n_src][d], v [S][n_src][64] bf16; w_q [d][3]; nbr [n_dst][n_nbr]
// (n_nbr <= 16), rel [n_dst][n_nbr][3]; out [S][n_dst][64] float32;
// kappa: workspace of S*n_src float4.
hipError_t launch_interp(const uint16_t* k, const uint16_t* v, const float* w_q, const int32_t* nbr,
                         const float* rel, long long slices, int n_src, int n_dst, int n_nbr, int d, float* out,
                         float4* kappa, hipStream_t stream);

// Bytes of the static device scratch that mosaic_bsa_forward_noalloc uses as
// its workspace (bsa_scratch.hip), and the current device's address of it
// (looked up once per device).
constexpr size_t kScratchBytes = size_t(256) << 20;
hipError_t scratch_buffer(void** ptr);

// largest m = N/block the backward's inverted-selection kernel holds in LDS
constexpr int kIndexMaxBlocks = 16384;

hipError_t launch_backward(const BwdLaunch& L, hipStream_t stream);

}  // namespace mosaic
