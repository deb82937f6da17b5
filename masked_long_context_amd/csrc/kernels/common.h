// Device helpers for the gfx950 kernels (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../tiling.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace bdattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;

// v_mfma_f32_32x32x16_bf16.  Operand lane layout (l = lane, g = l / 32):
//   A (32 x 16): lane holds row l % 32, k = 8g .. 8g + 7
//   B (16 x 32): lane holds col l % 32, k = 8g .. 8g + 7
//   C (32 x 32): lane holds col l % 32, rows 8 (r / 4) + 4 g + r % 4 for r = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of k-index kk (0..7) of lane group g inside a 16-chunk, when the
// operand comes straight from the C registers of a previous 32x32 MFMA:
// C regs 8c..8c+7 of group g hold rows 16c + {4g..4g+3, 8+4g..8+4g+3}.
// Memory copies of the other operand store a 16-chunk in this order, so that a
// lane reads its 8 values with one 16-byte load.  The map swaps bits 2 and 3.
__host__ __device__ __forceinline__ int perm16(int pos) {
  return (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ u32x4 ld_u32x4(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st_u32x4(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// 8 fp32 values (C regs r0 .. r0 + 7) -> bf16x8 B operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x16 &c, int r0) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)c[r0 + i];
  return o;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// K and V buffers holding row r (wave-uniform) of key segment s, and r's row in
// them.  SPLIT: segment 0 sits in the buffers of a.sh; otherwise every segment
// is one buffer (a.k[s], a.v[s]) and no lookup is made.
template <bool SPLIT, class Args>
__device__ __forceinline__ int seg_buffer(const Args &a, int s, int r, const void *&k, const void *&v) {
  if (SPLIT && s == 0) {
    const int i = min(r / a.sh.len, a.sh.n - 1);
    k = a.sh.k[i];
    v = a.sh.v[i];
    return r - i * a.sh.len;
  }
  k = a.k[s];
  v = a.v[s];
  return r;
}

// The same for the dK and dV buffers (backward).
template <bool SPLIT, class Args>
__device__ __forceinline__ int grad_buffer(const Args &a, int s, int r, void *&dk, void *&dv) {
  if (SPLIT && s == 0) {
    const int i = min(r / a.sh.len, a.sh.n - 1);
    dk = a.gsh.dk[i];
    dv = a.gsh.dv[i];
    return r - i * a.sh.len;
  }
  dk = a.dk[s];
  dv = a.dv[s];
  return r;
}

// Read of a table that no kernel writes while it runs, through the constant
// address space: with a uniform address this becomes a scalar (SMEM) load,
// which waits on lgkmcnt and so never stalls behind in-flight vector loads.
// Marks a branch the compiler must keep: code that contains it is never
// speculated into straight-line selects.  Used on the rare partial-tile masks,
// which would otherwise run on every tile.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::); }

template <class T>
__device__ __forceinline__ T ld_table(const T *p, int64_t i) {
  return ((const __attribute__((address_space(4))) T *)p)[i];
}

}  // namespace bdattn
