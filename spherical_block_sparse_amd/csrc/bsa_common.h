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

#include <type_traits>

#include "bsa_launch.h"

namespace mosaic {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

// word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// no swizzle, stride 0 (offsets are plain byte offsets, range-checked
// against the record count)
constexpr int kRsrcWord3 = 0x00020000;

// Direct loads into LDS (lane l's 16 bytes land at M0 + 16*l), written as
// inline assembly so that the compiler does not track them: it would
// otherwise make every transposing LDS read wait for all loads in flight
// (it cannot tell which buffer those reads touch), which serialises the
// prefetch of the next chunk with the current one.  The loads have no
// register results; their completion is awaited explicitly (s_waitcnt
// vmcnt, then a barrier) before a buffer is read.  M0 is restored.  A
// scalar write of M0 needs one wait state before an LDS-DMA load reads it
// (the compiler cannot insert it inside the assembly), hence the s_nop 0.
typedef int int32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of p as a scalar (the asm operands below must be SGPRs;
// every caller passes a workgroup-uniform address)
__device__ __forceinline__ int lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((int)(unsigned)(uintptr_t)(lds_void*)p);
}

__device__ __forceinline__ void dma_buffer(const void* lds, int voff, int32x4 rsrc, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(lds)), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

__device__ __forceinline__ void dma_global(const void* lds, const void* src) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(lds)), "v"(src)
      : "memory");
}

// The same two loads with the LDS destination given as a scalar base plus a
// compile-time byte offset, added to M0 inside the asm.  A loop that issues
// many loads into a few buffers then keeps one base register live instead of
// one hoisted address per load (which spills scalar registers).
template <int OFF>
__device__ __forceinline__ void dma_buffer_at(int lds_base, int voff, int32x4 rsrc, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(OFF)
      : "memory", "scc");
}

template <int OFF>
__device__ __forceinline__ void dma_global_at(int lds_base, const void* src) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(src), "n"(OFF)
      : "memory", "scc");
}

// The same for two loads sharing one M0 save and restore: K and V rows at
// the same per-lane offset into two buffers (OFF0, OFF1 bytes past lds_base).
template <int OFF0, int OFF1>
__device__ __forceinline__ void dma_buffer_pair_at(int lds_base, int voff, int32x4 r0, int32x4 r1, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %5 offen lds\n\t"
      "s_add_u32 m0, %1, %7\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(r0), "s"(r1), "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(OFF0),
        "n"(OFF1)
      : "memory", "scc");
}

template <int OFF0, int OFF1>
__device__ __forceinline__ void dma_global_pair_at(int lds_base, const void* src0, const void* src1) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(src0), "v"(src1), "n"(OFF0), "n"(OFF1)
      : "memory", "scc");
}

// calls f(std::integral_constant<int, i>) for i = I .. N-1, so that i can
// feed a template argument
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// buffer resource of one slice's tensor: base, stride 0, byte range, word 3
__device__ __forceinline__ int32x4 slice_rsrc(const void* base, int bytes) {
  const unsigned long long b = (unsigned long long)base;
  int32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffull));
  r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffull));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcWord3;
  return r;
}


}  // namespace mosaic
