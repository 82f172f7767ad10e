// C-ABI entry points of libmosaic_bsa (declared in include/mosaic_bsa.h).
//
// Every entry point validates all arguments before the first HIP call, so an
// invalid call launches nothing and leaves the outputs untouched; errors are
// returned as mosaic_status with a thread-local message.
#include "mosaic_bsa.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>

#include "bsa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

mosaic_status fail(mosaic_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

mosaic_status ok() {
  g_last_error[0] = '\0';
  return MOSAIC_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Shape {
  long long slices;
  int n_tok;
  int m;
  int d;
  int block;
  int topn;
  int window;   // clipped to 2N (a wider window sees the same keys)
};

enum : unsigned { kUsesTopn = 1, kUsesWindow = 2 };

// Checks the sizes shared by every entry point; `uses` says whether this
// entry point takes topn and window.
mosaic_status check_shape(int batch, int heads, int head_dim, int nside, int block, int topn,
                          int window, unsigned uses, Shape* s) {
  if (batch < 1 || heads < 1) return fail(MOSAIC_ERR_BAD_SHAPE, "batch (%d) and heads (%d) must be >= 1", batch, heads);
  if (nside < 1 || (nside & (nside - 1)))
    return fail(MOSAIC_ERR_BAD_SHAPE, "nside (%d) must be a power of two >= 1", nside);
  if (nside > 8192) return fail(MOSAIC_ERR_UNSUPPORTED, "nside %d: N = 12*nside^2 must fit in int32", nside);
  const long long n_tok = 12LL * nside * nside;
  if (block < 1 || (block & (block - 1)) || (__builtin_ctz((unsigned)block) & 1))
    return fail(MOSAIC_ERR_BAD_SHAPE, "block (%d) must be a power of four", block);
  if ((long long)block > (long long)nside * nside)
    return fail(MOSAIC_ERR_BAD_SHAPE, "block (%d) must be <= nside^2 (%lld) so it is one coarse pixel", block,
                (long long)nside * nside);
  const long long m = n_tok / block;
  if ((uses & kUsesTopn) && (topn < 1 || topn > m))
    return fail(MOSAIC_ERR_BAD_SHAPE, "topn (%d) must lie in [1, m=%lld]", topn, m);
  if ((uses & kUsesWindow) && window < 1) return fail(MOSAIC_ERR_BAD_SHAPE, "window (%d) must be >= 1", window);
  if (head_dim != 32 && head_dim != 64)
    return fail(MOSAIC_ERR_UNSUPPORTED, "head_dim %d: supported head_dim is 32 or 64", head_dim);
  const long long slices = (long long)batch * heads;
  // One-dimensional grids whose work-item count must fit in 32 bits: the
  // tiled fine kernel launches 2 work-items per token, the selection 4 per
  // block and the pooling 24 per block; the one-wave kernels for blocks of
  // 1 or 4 tokens or top-n above 64 launch 64 per query (fine) or per
  // query block (selection).
  const bool big_topn = (uses & kUsesTopn) && topn > 64;
  long long items = 24 * slices * m;
  if (block < 16 || big_topn) items = 64 * slices * n_tok;
  if (slices * n_tok > 0x7fffffffLL || items > 0xffffffffLL)
    return fail(MOSAIC_ERR_UNSUPPORTED, "batch*heads*N too large for one launch");
  s->slices = slices;
  s->n_tok = (int)n_tok;
  s->m = (int)m;
  s->d = head_dim;
  s->block = block;
  s->topn = (uses & kUsesTopn) ? topn : 0;
  s->window = (uses & kUsesWindow) ? (int)((long long)window > 2 * n_tok ? 2 * n_tok : window) : 0;
  return MOSAIC_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
  size_t qbar, kbar, vbar, ocg, knorm, kpieces, kbn2, selmax, total;
};

Workspace layout(const Shape& s) {
  const size_t e = (size_t)s.slices * s.m * s.d;
  Workspace w;
  w.qbar = 0;
  w.kbar = w.qbar + align256(e * sizeof(double));
  w.vbar = w.kbar + align256(e * sizeof(double));
  w.ocg = w.vbar + align256(e * sizeof(float));
  w.knorm = w.ocg + align256(e * sizeof(float));
  w.kpieces = w.knorm + align256((size_t)s.slices * s.m * sizeof(float));
  w.kbn2 = w.kpieces + align256(e * 2 * sizeof(uint16_t));
  w.selmax = w.kbn2 + align256((size_t)s.slices * s.m * sizeof(float));
  w.total = w.selmax + align256((size_t)s.slices * s.m * sizeof(float));
  return w;
}

// State the training forward leaves for the backward: the branch outputs
// and log2-sum-exps of the fine kernel, then the pooled rows and the
// compressed output (in the forward's own workspace layout).
struct Saved {
  size_t o, lse, pooled, total;
};

Saved saved_layout(const Shape& s) {
  const size_t en = (size_t)s.slices * s.n_tok;
  Saved v;
  v.o = 0;
  v.lse = align256(en * 2 * s.d * sizeof(float));
  v.pooled = v.lse + align256(en * 2 * sizeof(float));
  v.total = v.pooled + layout(s).total;
  return v;
}

// Backward workspace: recomputed forward pieces, bf16 copies, per-query
// statistics, pooled gradients and the inverted selection.
struct BwdWorkspace {
  size_t qbar, kbar, vbar, ocg, sel, dob, dob_loc, docg, docg_b, qbar_b, kbar_b, vbar_b, stats, stats_cg, dqbar, dkbar,
      dvbar, inv_off, inv_tmp, inv_list, total;
};

BwdWorkspace bwd_layout(const Shape& s) {
  const size_t em = (size_t)s.slices * s.m * s.d, en = (size_t)s.slices * s.n_tok * s.d;
  BwdWorkspace w;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o += align256(bytes); return r; };
  w.qbar = take(em * sizeof(double));
  w.kbar = take(em * sizeof(double));
  w.vbar = take(em * sizeof(float));
  w.ocg = take(em * sizeof(float));
  w.sel = take((size_t)s.slices * s.m * s.topn * sizeof(int32_t));
  w.dob = take(en * sizeof(uint16_t));
  w.dob_loc = take(en * sizeof(uint16_t));
  w.docg = take(em * sizeof(float));
  w.docg_b = take(em * sizeof(uint16_t));
  w.qbar_b = take(em * sizeof(uint16_t));
  w.kbar_b = take(em * sizeof(uint16_t));
  w.vbar_b = take(em * sizeof(uint16_t));
  w.stats = take((size_t)2 * s.slices * 3 * s.n_tok * sizeof(float));
  w.stats_cg = take((size_t)2 * s.slices * 3 * s.m * sizeof(float));
  w.dqbar = take(em * sizeof(float));
  w.dkbar = take(em * sizeof(float));
  w.dvbar = take(em * sizeof(float));
  w.inv_off = take((size_t)s.slices * (s.m + 1) * sizeof(int32_t));
  w.inv_tmp = take((size_t)s.slices * s.m * s.topn * sizeof(int32_t));
  w.inv_list = take((size_t)s.slices * s.m * s.topn * sizeof(int32_t));
  w.total = o;
  return w;
}

// what the backward kernels implement beyond the forward's own limits
mosaic_status check_backward_shape(const Shape& s) {
  if (s.block < 64) return fail(MOSAIC_ERR_UNSUPPORTED, "backward: block %d, the kernels need block >= 64", s.block);
  if (s.topn > 64) return fail(MOSAIC_ERR_UNSUPPORTED, "backward: topn %d, the kernels take at most 64", s.topn);
  if (s.m % 64) return fail(MOSAIC_ERR_UNSUPPORTED, "backward: m = N/block = %d must be a multiple of 64", s.m);
  if (s.m > mosaic::kIndexMaxBlocks)
    return fail(MOSAIC_ERR_UNSUPPORTED, "backward: m = N/block = %d, at most %d blocks", s.m, mosaic::kIndexMaxBlocks);
  return MOSAIC_OK;
}

mosaic_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOSAIC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// encoder layer: limits of the projection kernels and the workspace
mosaic_status check_layer(const Shape& s, int heads, int channels) {
  if (channels < 64 || channels % 64 || channels > 16384)
    return fail(MOSAIC_ERR_UNSUPPORTED, "channels %d: the projections need a multiple of 64 in [64, 16384]",
                channels);
  if ((heads * s.d) % 64)
    return fail(MOSAIC_ERR_UNSUPPORTED, "heads*head_dim = %d: the output projection needs a multiple of 64",
                heads * s.d);
  return MOSAIC_OK;
}

struct LayerWorkspace {
  size_t q, k, v, gates, attn, bsa, total;
};

LayerWorkspace layer_layout(const Shape& s) {
  const size_t e = (size_t)s.slices * s.n_tok * s.d;
  LayerWorkspace w;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o += align256(bytes); return r; };
  w.q = take(e * sizeof(uint16_t));
  w.k = take(e * sizeof(uint16_t));
  w.v = take(e * sizeof(uint16_t));
  w.gates = take((size_t)s.slices * s.n_tok * 3 * sizeof(float));
  w.attn = take(e * sizeof(uint16_t));   // bf16 [b][N][H][d], the heads side by side
  w.bsa = take(layout(s).total);
  w.total = o;
  return w;
}


// The selected branch's score bound per query block, for the tiled fine
// kernel only (the one-wave kernels do not use it).
hipError_t sel_bound(const Shape& s, const int32_t* sel_idx, const float* knorm, float* selmax, hipStream_t hs) {
  if (!mosaic::fine_tiled(s.n_tok, s.block, s.topn)) return hipSuccess;
  return mosaic::launch_sel_bound(sel_idx, knorm, selmax, s.slices, s.m, s.topn, hs);
}

// The forward's three launches on a validated shape, with the workspace at ws
// (layout(s).total bytes, 256-byte aligned).
mosaic_status run_forward(const Shape& s, const void* q, const void* k, const void* v, const float* gates,
                          float* out, int32_t* sel_idx, char* ws, hipStream_t hs) {
  const Workspace w = layout(s);
  double* qbar = reinterpret_cast<double*>(ws + w.qbar);
  double* kbar = reinterpret_cast<double*>(ws + w.kbar);
  float* vbar = reinterpret_cast<float*>(ws + w.vbar);
  float* ocg = reinterpret_cast<float*>(ws + w.ocg);
  float* knorm = reinterpret_cast<float*>(ws + w.knorm);
  uint16_t* kpieces = reinterpret_cast<uint16_t*>(ws + w.kpieces);
  float* kbn2 = reinterpret_cast<float*>(ws + w.kbn2);
  hipError_t e = mosaic::launch_pool(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), qbar, kbar, vbar, s.slices, s.n_tok,
                                     s.d, s.block, hs, knorm, kpieces, kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_pool launch");
  e = mosaic::launch_compress_select(qbar, kbar, vbar, ocg, sel_idx, s.slices, s.m, s.d, s.topn, hs, kpieces,
                                     kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_compress_select launch");
  float* selmax = reinterpret_cast<float*>(ws + w.selmax);
  if ((e = sel_bound(s, sel_idx, knorm, selmax, hs)) != hipSuccess) return hip_status(e, "selection bound launch");
  e = mosaic::launch_fine(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), gates, ocg, sel_idx, out, s.slices, s.n_tok, s.d,
                          s.block, s.topn, s.window, hs, knorm, nullptr, nullptr, nullptr, 1, selmax);
  return hip_status(e, "bsa_fine launch");
}

#define REQUIRE_PTR(p) \
  if (!(p)) return fail(MOSAIC_ERR_NULL_POINTER, "%s is NULL", #p)
#define REQUIRE_ALIGN(p, a) \
  if (!aligned((p), (a))) return fail(MOSAIC_ERR_MISALIGNED, "%s is not %d-byte aligned", #p, (int)(a))

}  // namespace

extern "C" {

int mosaic_bsa_abi_version(void) { return MOSAIC_BSA_ABI_VERSION; }

const char* mosaic_status_string(int status) {
  switch (status) {
    case MOSAIC_OK: return "MOSAIC_OK";
    case MOSAIC_ERR_NULL_POINTER: return "MOSAIC_ERR_NULL_POINTER";
    case MOSAIC_ERR_BAD_SHAPE: return "MOSAIC_ERR_BAD_SHAPE";
    case MOSAIC_ERR_UNSUPPORTED: return "MOSAIC_ERR_UNSUPPORTED";
    case MOSAIC_ERR_MISALIGNED: return "MOSAIC_ERR_MISALIGNED";
    case MOSAIC_ERR_WORKSPACE: return "MOSAIC_ERR_WORKSPACE";
    case MOSAIC_ERR_HIP: return "MOSAIC_ERR_HIP";
    default: return "MOSAIC_ERR_UNKNOWN";
  }
}

const char* mosaic_last_error(void) { return g_last_error; }

size_t mosaic_bsa_workspace_bytes(int batch, int heads, int head_dim, int nside, int block, int topn) {
  Shape s;
  if (check_shape(batch, heads, head_dim, nside, block, topn, 0, kUsesTopn, &s) != MOSAIC_OK) return 0;
  return layout(s).total;
}

mosaic_status mosaic_bsa_pool(const void* q, const void* k, const void* v, int batch, int heads,
                              int head_dim, int nside, int block, double* qbar, double* kbar,
                              float* vbar, float* knorm, uint16_t* kpieces, float* kbn2, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v);
  REQUIRE_PTR(qbar); REQUIRE_PTR(kbar); REQUIRE_PTR(vbar);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16);
  REQUIRE_ALIGN(qbar, 16); REQUIRE_ALIGN(kbar, 16); REQUIRE_ALIGN(vbar, 16); REQUIRE_ALIGN(knorm, 4);
  REQUIRE_ALIGN(kpieces, 16); REQUIRE_ALIGN(kbn2, 4);
  if ((kpieces == nullptr) != (kbn2 == nullptr))
    return fail(MOSAIC_ERR_NULL_POINTER, "kpieces and kbn2 are given together or not at all");
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, 0, 0, 0, &s);
  if (st != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_pool(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), qbar, kbar, vbar, s.slices,
                                        s.n_tok, s.d, s.block, static_cast<hipStream_t>(stream), knorm, kpieces,
                                        kbn2),
                    "bsa_pool launch");
}

mosaic_status mosaic_bsa_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                         int batch, int heads, int head_dim, int nside, int block,
                                         int topn, const uint16_t* kpieces, const float* kbn2, float* o_cg,
                                         int32_t* sel_idx, void* stream) {
  REQUIRE_PTR(qbar); REQUIRE_PTR(kbar); REQUIRE_PTR(vbar); REQUIRE_PTR(o_cg); REQUIRE_PTR(sel_idx);
  REQUIRE_ALIGN(qbar, 16); REQUIRE_ALIGN(kbar, 16); REQUIRE_ALIGN(vbar, 16); REQUIRE_ALIGN(o_cg, 16);
  REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(kpieces, 16); REQUIRE_ALIGN(kbn2, 4);
  if ((kpieces == nullptr) != (kbn2 == nullptr))
    return fail(MOSAIC_ERR_NULL_POINTER, "kpieces and kbn2 are given together or not at all");
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, 0, kUsesTopn, &s);
  if (st != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_compress_select(qbar, kbar, vbar, o_cg, sel_idx, s.slices, s.m, s.d,
                                                   s.topn, static_cast<hipStream_t>(stream), kpieces, kbn2),
                    "bsa_compress_select launch");
}

mosaic_status mosaic_bsa_fine(const void* q, const void* k, const void* v, const float* gates,
                              const float* o_cg, const int32_t* sel_idx, const float* knorm,
                              const float* sel_bound, int batch, int heads, int head_dim, int nside, int block,
                              int topn, int window, float* out, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates); REQUIRE_PTR(o_cg);
  REQUIRE_PTR(sel_idx); REQUIRE_PTR(out);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  REQUIRE_ALIGN(o_cg, 16); REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(knorm, 4);
  REQUIRE_ALIGN(sel_bound, 4);
  if (sel_bound && !knorm) return fail(MOSAIC_ERR_NULL_POINTER, "sel_bound is given without knorm");
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_fine(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), gates, o_cg, sel_idx, out,
                                        s.slices, s.n_tok, s.d, s.block, s.topn, s.window,
                                        static_cast<hipStream_t>(stream), knorm, nullptr, nullptr, nullptr, 1,
                                        sel_bound),
                    "bsa_fine launch");
}

mosaic_status mosaic_bsa_select_bound(const int32_t* sel_idx, const float* knorm, int batch, int heads,
                                      int head_dim, int nside, int block, int topn, float* sel_bound,
                                      void* stream) {
  REQUIRE_PTR(sel_idx); REQUIRE_PTR(knorm); REQUIRE_PTR(sel_bound);
  REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(knorm, 4); REQUIRE_ALIGN(sel_bound, 4);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, 0, kUsesTopn, &s);
  if (st != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_sel_bound(sel_idx, knorm, sel_bound, s.slices, s.m, s.topn,
                                             static_cast<hipStream_t>(stream)),
                    "selection bound launch");
}

mosaic_status mosaic_bsa_forward(const void* q, const void* k, const void* v, const float* gates,
                                 int batch, int heads, int head_dim, int nside, int block, int topn,
                                 int window, float* out, int32_t* sel_idx, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates); REQUIRE_PTR(out);
  REQUIRE_PTR(sel_idx); REQUIRE_PTR(workspace);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(workspace, 256);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  const Workspace w = layout(s);
  if (workspace_bytes < w.total)
    return fail(MOSAIC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, w.total);
  return run_forward(s, q, k, v, gates, out, sel_idx, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mosaic_status mosaic_bsa_forward_noalloc(const void* q, const void* k, const void* v, const float* gates,
                                         int batch, int heads, int head_dim, int nside, int block, int topn,
                                         int window, float* out, int32_t* sel_idx, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates); REQUIRE_PTR(out); REQUIRE_PTR(sel_idx);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(sel_idx, 4);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  const Workspace w = layout(s);
  if (w.total > mosaic::kScratchBytes)
    return fail(MOSAIC_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of workspace; the static scratch holds %zu (use mosaic_bsa_forward)",
                w.total, mosaic::kScratchBytes);
  void* ws = nullptr;
  const hipError_t e = mosaic::scratch_buffer(&ws);
  if (e != hipSuccess) return hip_status(e, "static scratch lookup");
  return run_forward(s, q, k, v, gates, out, sel_idx, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// HEALPix coarsening

mosaic_status mosaic_healpix_coarsen(const void* x, int batch, int channels, int nside, int levels, float* y,
                                     void* stream) {
  REQUIRE_PTR(x); REQUIRE_PTR(y);
  REQUIRE_ALIGN(x, 16); REQUIRE_ALIGN(y, 16);
  if (batch < 1) return fail(MOSAIC_ERR_BAD_SHAPE, "batch (%d) must be >= 1", batch);
  if (nside < 1 || (nside & (nside - 1)))
    return fail(MOSAIC_ERR_BAD_SHAPE, "nside (%d) must be a power of two >= 1", nside);
  if (nside > 8192) return fail(MOSAIC_ERR_UNSUPPORTED, "nside %d: N = 12*nside^2 must fit in int32", nside);
  if (levels < 1 || (nside >> levels) < 1 || ((nside >> levels) << levels) != nside)
    return fail(MOSAIC_ERR_BAD_SHAPE, "levels (%d) must be >= 1 with nside / 2^levels >= 1", levels);
  if (channels < 8 || channels % 8)
    return fail(MOSAIC_ERR_UNSUPPORTED, "channels %d: the kernel needs a multiple of 8", channels);
  const long long n_tok = 12LL * nside * nside;
  if ((long long)batch * n_tok * channels / 8 > 0x7fffffffLL * 256LL)
    return fail(MOSAIC_ERR_UNSUPPORTED, "batch*N*channels too large for one launch");
  return hip_status(mosaic::launch_coarsen(static_cast<const uint16_t*>(x), y, batch, (int)n_tok, channels, levels,
                                           static_cast<hipStream_t>(stream)),
                    "healpix_coarsen launch");
}

// ---------------------------------------------------------------------------
// lat-lon -> HEALPix interpolation

size_t mosaic_interp_workspace_bytes(int slices, int n_src) {
  if (slices < 1 || n_src < 1) return 0;
  return align256((size_t)slices * n_src * 4 * sizeof(float));
}

mosaic_status mosaic_interp_attention(const void* k, const void* v, const float* w_q, const int32_t* nbr,
                                      const float* rel, int slices, int n_src, int n_dst, int n_nbr, int d, int dv,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(w_q); REQUIRE_PTR(nbr); REQUIRE_PTR(rel); REQUIRE_PTR(out);
  REQUIRE_PTR(workspace);
  REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(w_q, 4); REQUIRE_ALIGN(nbr, 4); REQUIRE_ALIGN(rel, 4);
  REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(workspace, 256);
  if (slices < 1 || n_src < 1 || n_dst < 1)
    return fail(MOSAIC_ERR_BAD_SHAPE, "slices (%d), n_src (%d) and n_dst (%d) must be >= 1", slices, n_src, n_dst);
  if (n_nbr < 1 || n_nbr > 16)
    return fail(MOSAIC_ERR_UNSUPPORTED, "n_nbr %d: the kernel takes 1 .. 16 neighbours per target", n_nbr);
  if (d < 8 || d > 256 || d % 8) return fail(MOSAIC_ERR_UNSUPPORTED, "d %d: a multiple of 8 in [8, 256]", d);
  if (dv != 64) return fail(MOSAIC_ERR_UNSUPPORTED, "dv %d: the kernel takes 64 value channels", dv);
  if ((long long)slices * n_src / 32 > 0x7fffffffLL || (long long)slices * n_dst / 16 > 0x7fffffffLL)
    return fail(MOSAIC_ERR_UNSUPPORTED, "slices*n_src or slices*n_dst too large for one launch");
  const size_t need = mosaic_interp_workspace_bytes(slices, n_src);
  if (workspace_bytes < need)
    return fail(MOSAIC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(mosaic::launch_interp(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), w_q, nbr,
                                          rel, slices, n_src, n_dst, n_nbr, d, out, static_cast<float4*>(workspace),
                                          static_cast<hipStream_t>(stream)),
                    "interpolation launch");
}

// ---------------------------------------------------------------------------
// encoder layer


size_t mosaic_bsa_layer_workspace_bytes(int batch, int heads, int head_dim, int channels, int nside, int block,
                                        int topn) {
  Shape s;
  if (check_shape(batch, heads, head_dim, nside, block, topn, 0, kUsesTopn, &s) != MOSAIC_OK) return 0;
  if (check_layer(s, heads, channels) != MOSAIC_OK) return 0;
  return layer_layout(s).total;
}

mosaic_status mosaic_bsa_layer_in(const void* x, const void* w_in, int batch, int heads, int head_dim,
                                  int channels, int nside, void* q, void* k, void* v, float* gates,
                                  void* stream) {
  REQUIRE_PTR(x); REQUIRE_PTR(w_in); REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates);
  REQUIRE_ALIGN(x, 16); REQUIRE_ALIGN(w_in, 16); REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16);
  REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, 16, 0, 0, 0, &s);
  if (st != MOSAIC_OK) return st;
  if ((st = check_layer(s, heads, channels)) != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_layer_in(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_in),
                                            batch, s.n_tok, channels, heads, s.d, static_cast<uint16_t*>(q),
                                            static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), gates,
                                            static_cast<hipStream_t>(stream)),
                    "layer input projection launch");
}

mosaic_status mosaic_bsa_layer_out(const float* attn, const void* w_out, const void* x, int batch, int heads,
                                   int head_dim, int channels, int nside, void* y, void* stream) {
  REQUIRE_PTR(attn); REQUIRE_PTR(w_out); REQUIRE_PTR(x); REQUIRE_PTR(y);
  REQUIRE_ALIGN(attn, 16); REQUIRE_ALIGN(w_out, 16); REQUIRE_ALIGN(x, 16); REQUIRE_ALIGN(y, 16);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, 16, 0, 0, 0, &s);
  if (st != MOSAIC_OK) return st;
  if ((st = check_layer(s, heads, channels)) != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_layer_out(attn, static_cast<const uint16_t*>(w_out),
                                             static_cast<const uint16_t*>(x), batch, s.n_tok, channels, heads, s.d,
                                             static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream)),
                    "layer output projection launch");
}

mosaic_status mosaic_bsa_layer_out_merged(const void* attn, const void* w_out, const void* x, int batch,
                                          int heads, int head_dim, int channels, int nside, void* y,
                                          void* stream) {
  REQUIRE_PTR(attn); REQUIRE_PTR(w_out); REQUIRE_PTR(x); REQUIRE_PTR(y);
  REQUIRE_ALIGN(attn, 16); REQUIRE_ALIGN(w_out, 16); REQUIRE_ALIGN(x, 16); REQUIRE_ALIGN(y, 16);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, 16, 0, 0, 0, &s);
  if (st != MOSAIC_OK) return st;
  if ((st = check_layer(s, heads, channels)) != MOSAIC_OK) return st;
  return hip_status(mosaic::launch_layer_out_merged(static_cast<const uint16_t*>(attn),
                                                    static_cast<const uint16_t*>(w_out),
                                                    static_cast<const uint16_t*>(x), batch, s.n_tok, channels,
                                                    heads, s.d, static_cast<uint16_t*>(y),
                                                    static_cast<hipStream_t>(stream)),
                    "layer output projection launch");
}

mosaic_status mosaic_bsa_layer_forward(const void* x, const void* w_in, const void* w_out, int batch, int heads,
                                       int head_dim, int channels, int nside, int block, int topn, int window,
                                       void* y, int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  REQUIRE_PTR(x); REQUIRE_PTR(w_in); REQUIRE_PTR(w_out); REQUIRE_PTR(y); REQUIRE_PTR(sel_idx);
  REQUIRE_PTR(workspace);
  REQUIRE_ALIGN(x, 16); REQUIRE_ALIGN(w_in, 16); REQUIRE_ALIGN(w_out, 16); REQUIRE_ALIGN(y, 16);
  REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(workspace, 256);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  if ((st = check_layer(s, heads, channels)) != MOSAIC_OK) return st;
  if (x == y) return fail(MOSAIC_ERR_BAD_SHAPE, "y must not alias x");
  const LayerWorkspace lw = layer_layout(s);
  if (workspace_bytes < lw.total)
    return fail(MOSAIC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, lw.total);
  char* ws = static_cast<char*>(workspace);
  uint16_t* q = reinterpret_cast<uint16_t*>(ws + lw.q);
  uint16_t* k = reinterpret_cast<uint16_t*>(ws + lw.k);
  uint16_t* v = reinterpret_cast<uint16_t*>(ws + lw.v);
  float* gates = reinterpret_cast<float*>(ws + lw.gates);
  uint16_t* attn = reinterpret_cast<uint16_t*>(ws + lw.attn);
  char* bws = ws + lw.bsa;
  const Workspace w = layout(s);
  double* qbar = reinterpret_cast<double*>(bws + w.qbar);
  double* kbar = reinterpret_cast<double*>(bws + w.kbar);
  float* vbar = reinterpret_cast<float*>(bws + w.vbar);
  float* ocg = reinterpret_cast<float*>(bws + w.ocg);
  float* knorm = reinterpret_cast<float*>(bws + w.knorm);
  uint16_t* kpieces = reinterpret_cast<uint16_t*>(bws + w.kpieces);
  float* kbn2 = reinterpret_cast<float*>(bws + w.kbn2);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = mosaic::launch_layer_in(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_in), batch,
                                         s.n_tok, channels, heads, s.d, q, k, v, gates, hs);
  if (e != hipSuccess) return hip_status(e, "layer input projection launch");
  e = mosaic::launch_pool(q, k, v, qbar, kbar, vbar, s.slices, s.n_tok, s.d, s.block, hs, knorm, kpieces, kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_pool launch");
  e = mosaic::launch_compress_select(qbar, kbar, vbar, ocg, sel_idx, s.slices, s.m, s.d, s.topn, hs, kpieces,
                                     kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_compress_select launch");
  float* selmax = reinterpret_cast<float*>(bws + w.selmax);
  if ((e = sel_bound(s, sel_idx, knorm, selmax, hs)) != hipSuccess) return hip_status(e, "selection bound launch");
  e = mosaic::launch_fine(q, k, v, gates, ocg, sel_idx, nullptr, s.slices, s.n_tok, s.d, s.block, s.topn, s.window,
                          hs, knorm, nullptr, nullptr, attn, heads, selmax);
  if (e != hipSuccess) return hip_status(e, "bsa_fine launch");
  return hip_status(mosaic::launch_layer_out_merged(attn, static_cast<const uint16_t*>(w_out),
                                                    static_cast<const uint16_t*>(x), batch, s.n_tok, channels, heads,
                                                    s.d, static_cast<uint16_t*>(y), hs),
                    "layer output projection launch");
}

size_t mosaic_bsa_saved_bytes(int batch, int heads, int head_dim, int nside, int block) {
  Shape s;
  if (check_shape(batch, heads, head_dim, nside, block, 0, 0, 0, &s) != MOSAIC_OK) return 0;
  return saved_layout(s).total;
}

mosaic_status mosaic_bsa_forward_train(const void* q, const void* k, const void* v, const float* gates,
                                       int batch, int heads, int head_dim, int nside, int block, int topn,
                                       int window, float* out, int32_t* sel_idx, void* saved,
                                       size_t saved_bytes, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates); REQUIRE_PTR(out);
  REQUIRE_PTR(sel_idx); REQUIRE_PTR(saved);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  REQUIRE_ALIGN(out, 16); REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(saved, 256);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  const Saved sv = saved_layout(s);
  if (saved_bytes < sv.total)
    return fail(MOSAIC_ERR_WORKSPACE, "saved buffer of %zu bytes, %zu needed", saved_bytes, sv.total);
  char* base = static_cast<char*>(saved);
  const Workspace w = layout(s);
  char* ws = base + sv.pooled;
  double* qbar = reinterpret_cast<double*>(ws + w.qbar);
  double* kbar = reinterpret_cast<double*>(ws + w.kbar);
  float* vbar = reinterpret_cast<float*>(ws + w.vbar);
  float* ocg = reinterpret_cast<float*>(ws + w.ocg);
  float* knorm = reinterpret_cast<float*>(ws + w.knorm);
  uint16_t* kpieces = reinterpret_cast<uint16_t*>(ws + w.kpieces);
  float* kbn2 = reinterpret_cast<float*>(ws + w.kbn2);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = mosaic::launch_pool(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), qbar, kbar, vbar, s.slices, s.n_tok,
                                     s.d, s.block, hs, knorm, kpieces, kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_pool launch");
  e = mosaic::launch_compress_select(qbar, kbar, vbar, ocg, sel_idx, s.slices, s.m, s.d, s.topn, hs, kpieces,
                                     kbn2);
  if (e != hipSuccess) return hip_status(e, "bsa_compress_select launch");
  float* selmax = reinterpret_cast<float*>(ws + w.selmax);
  if ((e = sel_bound(s, sel_idx, knorm, selmax, hs)) != hipSuccess) return hip_status(e, "selection bound launch");
  e = mosaic::launch_fine(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), gates, ocg, sel_idx, out, s.slices, s.n_tok, s.d,
                          s.block, s.topn, s.window, hs, knorm, reinterpret_cast<float*>(base + sv.o),
                          reinterpret_cast<float*>(base + sv.lse), nullptr, 1, selmax);
  return hip_status(e, "bsa_fine launch");
}

size_t mosaic_bsa_backward_workspace_bytes(int batch, int heads, int head_dim, int nside, int block, int topn) {
  Shape s;
  if (check_shape(batch, heads, head_dim, nside, block, topn, 0, kUsesTopn, &s) != MOSAIC_OK) return 0;
  if (check_backward_shape(s) != MOSAIC_OK) return 0;
  return bwd_layout(s).total;
}

mosaic_status mosaic_bsa_backward(const void* q, const void* k, const void* v, const float* gates,
                                  const int32_t* sel_idx, const float* dout, int batch, int heads, int head_dim,
                                  int nside, int block, int topn, int window, const void* saved,
                                  size_t saved_bytes, float* dq, float* dk, float* dv, float* dgates,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(gates); REQUIRE_PTR(sel_idx); REQUIRE_PTR(dout);
  REQUIRE_PTR(dq); REQUIRE_PTR(dk); REQUIRE_PTR(dv); REQUIRE_PTR(dgates); REQUIRE_PTR(workspace);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k, 16); REQUIRE_ALIGN(v, 16); REQUIRE_ALIGN(gates, 4);
  REQUIRE_ALIGN(sel_idx, 4); REQUIRE_ALIGN(dout, 16); REQUIRE_ALIGN(dq, 16); REQUIRE_ALIGN(dk, 16);
  REQUIRE_ALIGN(dv, 16); REQUIRE_ALIGN(dgates, 4); REQUIRE_ALIGN(workspace, 256);
  if (saved) REQUIRE_ALIGN(saved, 256);
  Shape s;
  mosaic_status st = check_shape(batch, heads, head_dim, nside, block, topn, window, kUsesTopn | kUsesWindow, &s);
  if (st != MOSAIC_OK) return st;
  if ((st = check_backward_shape(s)) != MOSAIC_OK) return st;
  const BwdWorkspace w = bwd_layout(s);
  if (workspace_bytes < w.total)
    return fail(MOSAIC_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, w.total);
  const Saved sv = saved_layout(s);
  if (saved && saved_bytes < sv.total)
    return fail(MOSAIC_ERR_WORKSPACE, "saved buffer of %zu bytes, %zu needed", saved_bytes, sv.total);
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  mosaic::BwdLaunch L;
  L.q = static_cast<const uint16_t*>(q);
  L.k = static_cast<const uint16_t*>(k);
  L.v = static_cast<const uint16_t*>(v);
  L.gates = gates;
  L.sel = sel_idx;
  L.dout = dout;
  L.dq = dq;
  L.dk = dk;
  L.dv = dv;
  L.dgates = dgates;
  L.head_dim = s.d;
  L.slices = s.slices;
  L.n_tok = s.n_tok;
  L.block = s.block;
  L.topn = s.topn;
  L.window = s.window;
  double* qbar = reinterpret_cast<double*>(ws + w.qbar);
  double* kbar = reinterpret_cast<double*>(ws + w.kbar);
  float* vbar = reinterpret_cast<float*>(ws + w.vbar);
  float* ocg = reinterpret_cast<float*>(ws + w.ocg);
  L.save_o = nullptr;
  L.save_lse = nullptr;
  if (saved) {   // the training forward's pooled rows, compressed output and branch state
    const char* sb = static_cast<const char*>(saved);
    const Workspace fw = layout(s);
    qbar = reinterpret_cast<double*>(const_cast<char*>(sb + sv.pooled + fw.qbar));
    kbar = reinterpret_cast<double*>(const_cast<char*>(sb + sv.pooled + fw.kbar));
    vbar = reinterpret_cast<float*>(const_cast<char*>(sb + sv.pooled + fw.vbar));
    ocg = reinterpret_cast<float*>(const_cast<char*>(sb + sv.pooled + fw.ocg));
    L.save_o = reinterpret_cast<const float*>(sb + sv.o);
    L.save_lse = reinterpret_cast<const float*>(sb + sv.lse);
  }
  L.qbar = qbar;
  L.kbar = kbar;
  L.vbar = vbar;
  L.o_cg = ocg;
  L.dob = reinterpret_cast<uint16_t*>(ws + w.dob);
  L.dob_loc = reinterpret_cast<uint16_t*>(ws + w.dob_loc);
  L.docg = reinterpret_cast<float*>(ws + w.docg);
  L.docg_b = reinterpret_cast<uint16_t*>(ws + w.docg_b);
  L.qbar_b = reinterpret_cast<uint16_t*>(ws + w.qbar_b);
  L.kbar_b = reinterpret_cast<uint16_t*>(ws + w.kbar_b);
  L.vbar_b = reinterpret_cast<uint16_t*>(ws + w.vbar_b);
  L.stats = reinterpret_cast<float*>(ws + w.stats);
  L.stats_cg = reinterpret_cast<float*>(ws + w.stats_cg);
  L.dqbar = reinterpret_cast<float*>(ws + w.dqbar);
  L.dkbar = reinterpret_cast<float*>(ws + w.dkbar);
  L.dvbar = reinterpret_cast<float*>(ws + w.dvbar);
  L.inv_off = reinterpret_cast<int32_t*>(ws + w.inv_off);
  L.inv_tmp = reinterpret_cast<int32_t*>(ws + w.inv_tmp);
  L.inv_list = reinterpret_cast<int32_t*>(ws + w.inv_list);
  if (!saved) {
    // recompute the forward's pooling and compressed branch (its own
    // selection goes to scratch: the backward uses the caller's)
    hipError_t e = mosaic::launch_pool(L.q, L.k, L.v, qbar, kbar, vbar, s.slices, s.n_tok, s.d, s.block, hs);
    if (e != hipSuccess) return hip_status(e, "bsa_pool launch");
    e = mosaic::launch_compress_select(qbar, kbar, vbar, ocg, reinterpret_cast<int32_t*>(ws + w.sel), s.slices,
                                       s.m, s.d, s.topn, hs);
    if (e != hipSuccess) return hip_status(e, "bsa_compress_select launch");
  }
  return hip_status(mosaic::launch_backward(L, hs), "bsa_backward launch");
}

}  // extern "C"
