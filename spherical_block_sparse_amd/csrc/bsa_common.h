// Internal declarations shared by the BSA kernels and the C-ABI host code.
// Target: gfx950 (CDNA4), wave64.
//
// MFMA lane layouts used below (measured on gfx950 with a one-wave probe):
//   v_mfma_f32_16x16x32_bf16 : A[m][k] -> lane m + 16*(k/8), element k%8;
//                              B[k][n] -> lane n + 16*(k/8), element k%8;
//                              C[m][n] -> lane n + 16*(m/4), register m%4.
//   v_mfma_f32_16x16x4_f32   : A[m][k] -> lane m + 16*k; B[k][n] -> lane n + 16*k;
//                              C[m][n] -> lane n + 16*(m/4), register m%4.
//   v_mfma_f64_16x16x4_f64   : A, B as the f32 variant;
//                              C[m][n] -> lane n + 16*(m%4), register m/4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mosaic {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

hipError_t launch_pool(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* qbar,
                       double* kbar, float* vbar, long long slices, int n_tok, int head_dim,
                       int block, hipStream_t stream);

hipError_t launch_compress_select(const double* qbar, const double* kbar, const float* vbar,
                                  float* o_cg, int32_t* sel, long long slices, int m, int head_dim,
                                  int topn, hipStream_t stream);

hipError_t launch_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gates,
                       const float* o_cg, const int32_t* sel, float* out, long long slices,
                       int n_tok, int head_dim, int block, int topn, int window,
                       hipStream_t stream);

}  // namespace mosaic
