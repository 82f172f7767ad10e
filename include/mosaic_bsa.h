/*
 * mosaic_bsa.h — C ABI of the MI355X (gfx950) forward pass of MOSAIC's
 * mesh-aligned block-sparse attention (BSA) over HEALPix NESTED tokens.
 *
 * Operation (papernotes.org ICML2026 notes on "(Sparse) Attention to the
 * Details", section 关键设计 › "Mesh-aligned Block-Sparse Attention (BSA)"):
 * for every (batch, head) slice, the N = 12*nside^2 tokens in NESTED order
 * are cut into m = N/block contiguous blocks (each one coarse HEALPix pixel,
 * by the 4p..4p+3 children rule of the "HEALPix + NESTED" item);
 *   q̄, k̄, v̄   = block means of q, k, v                       (pooling)
 *   s_ij       = q̄_i·k̄_j / sqrt(d)
 *   o_CG_i     = sum_j softmax_j(s_ij) v̄_j                     (compressed)
 *   sel_i      = the topn j with largest s_ij, ties to lower j  (selection,
 *                shared by every query of block i)
 *   o_FG_t     = softmax attention of q_t over all tokens of the blocks sel_i
 *   o_L_t      = softmax attention of q_t over keys [t-floor(W/2), t+ceil(W/2))
 *                clipped to [0, N)                              (local)
 *   out_t      = g_t0·o_CG_{t/block} + g_t1·o_FG_t + g_t2·o_L_t
 * Scale 1/sqrt(d) everywhere, no causal mask, every slice independent.
 *
 * Conventions for every entry point
 *   - Buffers are device pointers owned by the caller; the library allocates
 *     nothing and keeps no state.  Inputs are never written.
 *   - Layouts are dense row-major: q, k, v, out [batch][heads][N][head_dim];
 *     gates [batch][heads][N][3] = (g_CG, g_FG, g_L); sel_idx
 *     [batch][heads][m][topn]; pooled / per-block tensors [batch][heads][m][head_dim].
 *   - q, k, v are bfloat16 bit patterns (uint16, round-to-nearest-even
 *     conversion done by the caller); gates, out and pooled v̄ / o_CG are
 *     float32; pooled q̄, k̄ are float64 (exact block means of bf16 data).
 *   - stream is a hipStream_t (NULL = the legacy default stream).  Every call
 *     only enqueues work and returns; faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated before any HIP call.  On error nothing is
 *     launched, outputs are untouched, and the status is returned; the text
 *     of the last error of the calling thread is mosaic_last_error().
 *   - Supported: nside a power of two with N < 2^31; block = 4^k with
 *     1 <= block <= nside^2 (so a block never straddles two base pixels);
 *     1 <= topn <= m; window >= 1; head_dim in {32, 64}; batch, heads >= 1;
 *     batch*heads*N < 2^31 (and below 2^26 when block < 16 or topn > 64,
 *     whose kernels run one wave per query).  Other head_dim values and
 *     larger sizes return MOSAIC_ERR_UNSUPPORTED.  Blocks of at least 16
 *     tokens with topn <= 64 take the tiled kernels; blocks of 1 or 4
 *     tokens and larger topn take one-wave-per-row kernels (same results,
 *     slower).
 *   - Alignment: q, k, v, out, o_cg, pooled buffers and sel_idx rows of 16
 *     bytes; gates 4 bytes; workspace 256 bytes.
 */
#ifndef MOSAIC_BSA_H
#define MOSAIC_BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOSAIC_BSA_ABI_VERSION 12

typedef enum mosaic_status {
  MOSAIC_OK = 0,
  MOSAIC_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  MOSAIC_ERR_BAD_SHAPE = 2,    /* sizes violate the definition (nside, block, topn, window) */
  MOSAIC_ERR_UNSUPPORTED = 3,  /* valid BSA, but outside what the kernels implement */
  MOSAIC_ERR_MISALIGNED = 4,   /* a pointer is not aligned as required */
  MOSAIC_ERR_WORKSPACE = 5,    /* workspace smaller than mosaic_bsa_workspace_bytes() */
  MOSAIC_ERR_HIP = 6           /* the HIP runtime refused a launch (no device, bad stream, ...) */
} mosaic_status;

/* Returns MOSAIC_BSA_ABI_VERSION of the built library. */
int mosaic_bsa_abi_version(void);

/* Static name of a status code ("MOSAIC_OK", ...). */
const char* mosaic_status_string(int status);

/* Text of the last failed call on the calling thread ("" if none). */
const char* mosaic_last_error(void);

/* Bytes of device workspace mosaic_bsa_forward needs: pooled q̄, k̄ (float64),
 * pooled v̄ and o_CG (float32), each [batch][heads][m][head_dim], then the
 * largest key norm of each block (float32 [batch][heads][m]), the bf16
 * pieces of k̄ ([batch][heads][m][2][head_dim]), |k̄_j|^2 (float32
 * [batch][heads][m]) and, per query block, the largest key norm over its
 * selected blocks (float32 [batch][heads][m]), 256-byte aligned sections.
 * Returns 0 if the shape is invalid or unsupported. */
size_t mosaic_bsa_workspace_bytes(int batch, int heads, int head_dim, int nside, int block, int topn);

/* The whole BSA forward pass (pool -> compressed + selection -> selected and
 * local fine attention with the gated sum), three kernels on `stream` (with
 * a small fourth between the last two that forms each query block's
 * selected-branch score bound, and the selection's float64 redo launch).
 *   q, k, v   in : bf16 bits [batch][heads][N][head_dim]
 *   gates     in : float32 [batch][heads][N][3]
 *   out       out: float32 [batch][heads][N][head_dim]
 *   sel_idx   out: int32 [batch][heads][m][topn], block indices in ascending order
 *   workspace in/out scratch of at least mosaic_bsa_workspace_bytes(...) bytes
 * (papernotes.org ICML2026 notes, 关键设计 › Mesh-aligned Block-Sparse Attention) */
mosaic_status mosaic_bsa_forward(const void* q, const void* k, const void* v, const float* gates,
                                 int batch, int heads, int head_dim, int nside, int block, int topn,
                                 int window, float* out, int32_t* sel_idx, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* mosaic_bsa_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a static
 * device array of 256 MiB inside the library: each GPU the library runs
 * this on holds its own copy until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's copy.  Sizes whose
 * workspace (mosaic_bsa_workspace_bytes) exceeds 256 MiB return
 * MOSAIC_ERR_UNSUPPORTED before any HIP call: e.g. batch 2 x 16 heads at
 * nside 256 (177 MB) fit, batch 24 x 8 heads at nside 128 (1.06 GB) do
 * not.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams or
 * threads without ordering between them) race.  Arguments, outputs and
 * errors otherwise as for mosaic_bsa_forward. */
mosaic_status mosaic_bsa_forward_noalloc(const void* q, const void* k, const void* v, const float* gates,
                                         int batch, int heads, int head_dim, int nside, int block, int topn,
                                         int window, float* out, int32_t* sel_idx, void* stream);

/* Pooling only: q̄, k̄ (float64) and v̄ (float32), [batch][heads][m][head_dim],
 * the mean of each block's `block` consecutive NESTED tokens (the block
 * summaries of the BSA item; the mean is this library's reading of the
 * unspecified pooling).  knorm (may be NULL): float32 [batch][heads][m], the
 * largest key norm max_t |k_t| of each block (float32 sums of squares); not
 * part of the method, it lets mosaic_bsa_fine bound scores in advance.
 * kpieces, kbn2 (both NULL, or both given; not part of the method): k̄ as
 * two bf16 pieces, k1 = bf16(k̄) and k2 = bf16(k̄ - k1) (formed in float32),
 * uint16 bits [batch][heads][m][2][head_dim] with k1 first (16-byte
 * aligned), and |k̄_j|^2 of each block, float32 [batch][heads][m], rounded
 * up; mosaic_bsa_compress_select ranks on them.  One of the two without the
 * other: MOSAIC_ERR_NULL_POINTER. */
mosaic_status mosaic_bsa_pool(const void* q, const void* k, const void* v, int batch, int heads,
                              int head_dim, int nside, int block, double* qbar, double* kbar,
                              float* vbar, float* knorm, uint16_t* kpieces, float* kbn2, void* stream);

/* Compressed branch and top-n selection from pooled tensors: o_cg
 * [batch][heads][m][head_dim] float32 = sum_j softmax_j(q̄_i·k̄_j/sqrt(d)) v̄_j,
 * and sel_idx [batch][heads][m][topn] = the topn largest logits of each row,
 * ties to the lower block index, listed in ascending order.  The selection
 * matches a float64 evaluation of the logits except on rows whose n-th and
 * (n+1)-th logits differ by a few float64 ulps.
 * kpieces, kbn2: NULL, or mosaic_bsa_pool's outputs for the same k̄ (both or
 * neither, else MOSAIC_ERR_NULL_POINTER).  Without them the logits are
 * float64 dot products.  With them and topn <= 16, each row is ranked on
 * bf16-piece logits (error below 2^-12.5 |q̄_i| max_j |k̄_j|) and certified:
 * keys within twice that bound of the n-th value are rescored in float64,
 * and a row that cannot be certified is selected exactly from its float64
 * logits, so the selection is the same; o_cg is formed from the approximate logits (its weights are
 * rounded to bf16 either way).  Pieces that do not belong to k̄ void the
 * selection. */
mosaic_status mosaic_bsa_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                         int batch, int heads, int head_dim, int nside, int block,
                                         int topn, const uint16_t* kpieces, const float* kbn2, float* o_cg,
                                         int32_t* sel_idx, void* stream);

/* Selected-block and sliding-window fine attention plus the gated sum, from
 * q, k, v (bf16), gates, o_cg (per block, float32) and sel_idx (any topn
 * valid block indices per row, each in [0, m); order is irrelevant):
 * out = g_CG·o_cg[t/block] + g_FG·o_FG + g_L·o_L.  bf16 products with
 * float32 accumulation; attention weights are rounded to bf16 before they
 * multiply v.  knorm (may be NULL): mosaic_bsa_pool's largest key norm per
 * block.  With it, queries whose scores it bounds closely enough use the
 * bound c·|q|·knorm as the fixed softmax reference in place of a running
 * maximum (the same softmax up to rounding).  A knorm that understates a
 * norm by a factor f lets weights grow to 2^((f-1)·bound): pass the pool's
 * own output.  sel_bound (may be NULL; not part of the method): with knorm,
 * mosaic_bsa_select_bound's output for the same sel_idx and knorm, which
 * the tiled kernel then reads in place of gathering knorm over each query
 * block's selected blocks (the same results); given without knorm:
 * MOSAIC_ERR_NULL_POINTER.  Alignment of sel_bound: 4 bytes. */
mosaic_status mosaic_bsa_fine(const void* q, const void* k, const void* v, const float* gates,
                              const float* o_cg, const int32_t* sel_idx, const float* knorm,
                              const float* sel_bound, int batch, int heads, int head_dim, int nside, int block,
                              int topn, int window, float* out, void* stream);

/* The selected branch's score bound per query block (not part of the
 * method): sel_bound [batch][heads][m] float32 = the largest knorm over the
 * topn blocks sel_idx [batch][heads][m][topn] lists for that query block
 * (indices clamped into [0, m)), knorm [batch][heads][m] from
 * mosaic_bsa_pool.  mosaic_bsa_forward, mosaic_bsa_forward_train and
 * mosaic_bsa_layer_forward form it in their workspaces between the
 * selection and the fine kernel; with this call a caller of the stages does
 * the same for mosaic_bsa_fine.  head_dim, nside, block and topn are
 * validated as for mosaic_bsa_fine (head_dim enters nothing else).
 * Alignment: 4 bytes. */
mosaic_status mosaic_bsa_select_bound(const int32_t* sel_idx, const float* knorm, int batch, int heads,
                                      int head_dim, int nside, int block, int topn, float* sel_bound,
                                      void* stream);

/* ---- HEALPix coarsening ---------------------------------------------------
 * A field on the NESTED pixels at nside taken to nside / 2^levels
 * (papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED: the children of
 * pixel p are 4p .. 4p+3, so a coarse pixel's 4^levels descendants are one
 * contiguous run of rows; the encoder downsamples to a coarser grid).  The
 * coarse value is the mean of the descendants, summed in float64.
 *   x  in : bf16 bits [batch][12*nside^2][channels]
 *   y  out: float32 [batch][12*(nside>>levels)^2][channels]
 * channels a multiple of 8; levels >= 1 with nside >> levels >= 1.
 * Alignment: x and y 16 bytes. */
mosaic_status mosaic_healpix_coarsen(const void* x, int batch, int channels, int nside, int levels, float* y,
                                     void* stream);

/* ---- Lat-lon -> HEALPix cross-attention interpolation ---------------------
 * papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED: each HEALPix
 * target i attends over its neighbouring source points j with the relative
 * positions as queries, o_i = sum_{j in N_i} softmax_j(q_ij^T k_j/sqrt(d)) v_j;
 * here q_ij = w_q p_ij (this library's reading).
 *   k        in : bf16 bits [slices][n_src][d]     source keys
 *   v        in : bf16 bits [slices][n_src][dv]    source values (dv = 64)
 *   w_q      in : float32 [d][3]                  query map of the relative position
 *   nbr      in : int32 [n_dst][n_nbr]            source indices of each target
 *                 (1 <= n_nbr <= 16; values clamped into [0, n_src))
 *   rel      in : float32 [n_dst][n_nbr][3]       relative positions p_ij
 *   out      out: float32 [slices][n_dst][dv]
 *   workspace   : at least mosaic_interp_workspace_bytes(slices, n_src)
 * d a multiple of 8 in [8, 256].  Alignment: k, v, out 16 bytes, workspace
 * 256, the rest 4. */
size_t mosaic_interp_workspace_bytes(int slices, int n_src);
mosaic_status mosaic_interp_attention(const void* k, const void* v, const float* w_q, const int32_t* nbr,
                                      const float* rel, int slices, int n_src, int n_dst, int n_nbr, int d, int dv,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Encoder layer --------------------------------------------------------
 * The papernotes.org ICML2026 notes (关键设计) run several BSA layers at
 * native HEALPix resolution; they specify neither the projections nor how
 * the gates are produced.  This library's layer is the plain reading, with
 * x [batch][N][channels] and y of the same shape, both bf16:
 *   [q | k | v | z] = x w_inᵀ        w_in  bf16 [3*H*d + 3*H][channels]
 *       rows h*d + j of each of q, k, v give head h, dimension j;
 *       row 3*H*d + 3*h + r gives the gate logit of head h, branch r
 *       (0 compressed, 1 selected, 2 local)
 *   g = sigmoid(z)
 *   y = x + merge_heads(BSA(q, k, v, g)) w_outᵀ   w_out bf16 [channels][H*d]
 * q, k, v, the merged attention output and y are rounded to bf16 (nearest
 * even); products accumulate in float32.  channels and H*d must be
 * multiples of 64 (channels <= 16384), else MOSAIC_ERR_UNSUPPORTED.
 * Alignment: x, y, w_in, w_out, q, k, v, attn 16 bytes; gates 4. */

/* Workspace of mosaic_bsa_layer_forward (q, k, v, gates, the attention
 * output and the BSA forward's workspace), or 0 for invalid sizes. */
size_t mosaic_bsa_layer_workspace_bytes(int batch, int heads, int head_dim, int channels, int nside,
                                        int block, int topn);

/* One encoder layer: input projection, mosaic_bsa_forward's kernels, output
 * projection with the residual.  sel_idx receives the layer's selection
 * ([batch][heads][m][topn]); y must not alias x. */
mosaic_status mosaic_bsa_layer_forward(const void* x, const void* w_in, const void* w_out, int batch,
                                       int heads, int head_dim, int channels, int nside, int block,
                                       int topn, int window, void* y, int32_t* sel_idx, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* The input projection alone: q, k, v bf16 [batch][heads][N][head_dim] and
 * gates float32 [batch][heads][N][3] from x and w_in. */
mosaic_status mosaic_bsa_layer_in(const void* x, const void* w_in, int batch, int heads, int head_dim,
                                  int channels, int nside, void* q, void* k, void* v, float* gates,
                                  void* stream);

/* The output projection alone: y = x + merge_heads(attn) w_outᵀ, attn the
 * float32 [batch][heads][N][head_dim] attention output (rounded to bf16
 * before the product). */
mosaic_status mosaic_bsa_layer_out(const float* attn, const void* w_out, const void* x, int batch, int heads,
                                   int head_dim, int channels, int nside, void* y, void* stream);

/* The same output projection from the attention output in the layout the
 * layer's own fine kernel writes: attn bf16 [batch][N][heads*head_dim], the
 * heads side by side (feature h*d + j), already rounded.  This is the GEMM
 * that mosaic_bsa_layer_forward runs.  y = x + attn w_outᵀ, rounded to bf16;
 * y may be x itself (each element's residual is read before it is written).
 * Sizes, alignment and errors as for mosaic_bsa_layer_out. */
mosaic_status mosaic_bsa_layer_out_merged(const void* attn, const void* w_out, const void* x, int batch,
                                          int heads, int head_dim, int channels, int nside, void* y,
                                          void* stream);

/* Bytes of the state mosaic_bsa_forward_train leaves for mosaic_bsa_backward,
 * or 0 when the sizes are invalid or unsupported.  Layout (256-byte aligned
 * sections): float32 o_FG_t, o_L_t [batch][heads][N][2][head_dim] (each
 * normalised), float32 [batch][heads][N][2] their base-2 log-sum-exp of
 * q_t·k_u·log2(e)/sqrt(d), then the forward workspace of
 * mosaic_bsa_workspace_bytes (q̄, k̄, v̄, o_CG, largest key norm per block). */
size_t mosaic_bsa_saved_bytes(int batch, int heads, int head_dim, int nside, int block);

/* mosaic_bsa_forward for training: the same sel_idx and out (up to float32
 * rounding of the gated sum), plus the state above in `saved` (in place of the
 * workspace, at least mosaic_bsa_saved_bytes(...) bytes, 256-byte aligned),
 * so that the backward need not recompute the pooled tensors, the compressed
 * branch or the two fine branches' softmax statistics.  The papernotes.org
 * ICML2026 notes (关键设计) describe a model trained end to end; this is the
 * forward such training runs. */
mosaic_status mosaic_bsa_forward_train(const void* q, const void* k, const void* v, const float* gates,
                                       int batch, int heads, int head_dim, int nside, int block, int topn,
                                       int window, float* out, int32_t* sel_idx, void* saved,
                                       size_t saved_bytes, void* stream);

/* Workspace bytes mosaic_bsa_backward needs for these sizes, or 0 when the
 * sizes are invalid or outside what the backward implements. */
size_t mosaic_bsa_backward_workspace_bytes(int batch, int heads, int head_dim, int nside, int block,
                                           int topn);

/* Gradient of mosaic_bsa_forward's `out` with respect to q, k, v and the
 * gates, given dout = dL/dout.  The papernotes.org ICML2026 notes (关键设计 ›
 * Mesh-aligned Block-Sparse Attention) describe a model trained end to end;
 * the gradient is that of the forward with the selection sel_idx held fixed
 * (top-n is piecewise constant) and each pooled mean's gradient spread evenly
 * over its block.
 *   q, k, v   in : bf16 bits [batch][heads][N][head_dim] (the forward's inputs)
 *   gates     in : float32 [batch][heads][N][3]
 *   sel_idx   in : int32 [batch][heads][m][topn], the forward's selection
 *                  (any valid block indices; clamped into [0, m))
 *   dout      in : float32 [batch][heads][N][head_dim]
 *   saved     in : the state of mosaic_bsa_forward_train for the same q, k,
 *                  v, gates and sizes (and sel_idx its selection), and its
 *                  size in bytes; or NULL (saved_bytes ignored): the
 *                  backward then recomputes that state itself
 *   dq, dk, dv out: float32 [batch][heads][N][head_dim], overwritten
 *   dgates    out: float32 [batch][heads][N][3], overwritten
 *   workspace in/out scratch of at least mosaic_bsa_backward_workspace_bytes(...)
 * All launches go to `stream`.  Without `saved` the forward's pooling,
 * compressed branch and fine-branch statistics are recomputed.  bf16
 * products with float32 accumulation (dout is rounded to bf16 for the
 * products; D = dout·o uses it in float32).
 * Besides the forward's limits, block >= 64, topn <= 64 and m = N/block a
 * multiple of 64 and at most 16384 are needed (MOSAIC_ERR_UNSUPPORTED
 * otherwise).
 * Alignment: q, k, v, dout, dq, dk, dv 16 bytes; gates, sel_idx, dgates 4;
 * workspace and saved 256.  Errors as for the forward: nothing is launched
 * and the outputs are untouched. */
mosaic_status mosaic_bsa_backward(const void* q, const void* k, const void* v, const float* gates,
                                  const int32_t* sel_idx, const float* dout, int batch, int heads,
                                  int head_dim, int nside, int block, int topn, int window,
                                  const void* saved, size_t saved_bytes, float* dq, float* dk, float* dv,
                                  float* dgates, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOSAIC_BSA_H */
