// LDS tiles for the gfx950 attention kernels.
//
// A tile is 64 rows of a row-major bf16 matrix with D elements per row, copied
// from global memory straight into LDS by global_load_lds_dwordx4 (each lane
// of a wave moves 16 bytes; a wave-wide load fills 1 KB of LDS in lane order).
// The 16-byte chunks of row r sit at chunk ^ swz(r), with
//   swz(r) = 2 (r mod 4) + (r / 4 mod 2),
// which keeps both access patterns free of bank conflicts:
//   * row reads (ds_read_b128): 8 lanes read the same chunk of 8 consecutive
//     rows -> swz takes 8 distinct values;
//   * transpose reads (ds_read_b64_tr_b16): 16 lanes read 2 adjacent chunks
//     of 4 consecutive rows -> the 8 (row, chunk) slots are distinct mod 8.
//
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane i supplies the address
// of 4 consecutive elements of row i / 4 (columns 4 (i mod 4) .. +3) of a 4 x 16
// block, and lane j receives column j of that block (rows 0..3).  Two such reads
// give a lane the 8 k-values of a 32x32x16 MFMA operand taken down a column.
#pragma once
#include "common.h"

namespace bdattn {

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define BD_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define BD_LDS_V4I16(p) ((__attribute__((address_space(3))) v4i16 *)(p))

template <int D>
struct Tile {
  static constexpr int ROWS = 64;
  static constexpr int ROWB = 2 * D;            // bytes per row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int RPK = 1024 / ROWB;       // rows per wave-wide load
  static constexpr int LOADS = BYTES / 1024;    // wave-wide loads per tile
};

__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ tile_swz(row)) << 4);
}

// This wave's share of the asynchronous copy of 64 rows starting at `g` (a
// wave-uniform pointer; row stride `stride` elements, 64 * stride < 2^30).  Rows
// at or beyond `nvalid` re-read row nvalid - 1 (the caller masks them);
// nvalid >= 1.  `wave` must be wave-uniform.  Issues Tile<D>::LOADS / NW loads.
template <int D, int NW>
__device__ __forceinline__ void tile_load(char *lds, const bf16 *g, int stride, int nvalid, int wave, int lane) {
  constexpr int PER = Tile<D>::LOADS / NW;
  static_assert(Tile<D>::LOADS % NW == 0, "tile loads must split evenly over the waves");
  const char *gb = reinterpret_cast<const char *>(g);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int kb = wave * PER + i;
    const int row = kb * Tile<D>::RPK + lane / Tile<D>::CPR;
    const int c = (lane % Tile<D>::CPR) ^ tile_swz(row);
    const int rr = row < nvalid ? row : nvalid - 1;
    const uint32_t off = (uint32_t)(rr * stride + c * 8) * 2u;
    __builtin_amdgcn_global_load_lds(gb + off, BD_LDS(lds + kb * 1024), 16, 0, 0);
  }
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// 8 consecutive elements [col, col + 8) of one row (col a multiple of 8).
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const char *t, int row, int col) {
  return *reinterpret_cast<const bf16x8 *>(t + tile_off<D>(row, col >> 3));
}

// For a tile X[k][m] (rows k, columns m): the 32x32x16 MFMA operand whose lane
// row/column is m = 32 mt + lane % 32 and whose 8 k-values are the rows of
// 16-chunk c16 in the order the C registers of a previous MFMA hold them
// (rows 16 c16 + 4 g + 0..3, then 16 c16 + 8 + 4 g + 0..3, g = lane / 32).
template <int D>
__device__ __forceinline__ bf16x8 tile_tr8(const char *t, int c16, int mt, int lane) {
  const int i = lane & 15, G = lane >> 4;
  const int col = 32 * mt + 16 * (G & 1) + 4 * (i & 3);
  const int row = 16 * c16 + 4 * (G >> 1) + (i >> 2);
  const int sub = (col & 7) * 2;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BD_LDS_V4I16(t + tile_off<D>(row, col >> 3) + sub));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BD_LDS_V4I16(t + tile_off<D>(row + 8, col >> 3) + sub));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

// Row reads of a tile with a fixed lane pattern: row 32 t + (lane % 32), columns
// 16 c + 8 (lane / 32) .. +7 (the A/B operand of a 32x32x16 MFMA over the head
// dim).  For this lane, swz(row) = s is constant, and the physical chunk is
// (2c + g) ^ s = 2 (c ^ (s >> 1)) + (g ^ (s & 1)); with c = 4m + n only n sees
// the XOR, so four per-lane offsets (n = 0..3) plus immediates cover every read.
template <int D>
struct RowReader {
  int off[4];
  __device__ __forceinline__ explicit RowReader(int lane) {
    const int j = lane & 31, g = lane >> 5, sw = tile_swz(j);
#pragma unroll
    for (int n = 0; n < 4; ++n) off[n] = j * (2 * D) + 32 * (n ^ (sw >> 1)) + 16 * (g ^ (sw & 1));
  }
  __device__ __forceinline__ bf16x8 operator()(const char *t, int tb, int c) const {
    return *reinterpret_cast<const bf16x8 *>(t + off[c & 3] + 128 * (c >> 2) + tb * 32 * (2 * D));
  }
};

// Transpose reads (tile_tr8) with a fixed lane pattern.  Row bits 0..2 depend on
// the lane only, so s = swz(row) is constant; the chunk (4 mt + r) ^ s =
// 4 (mt ^ (s >> 2)) + (r ^ (s & 3)), and with mt = 2m + n only n sees the XOR:
// two per-lane offsets (n = 0, 1) plus immediates.
template <int D>
struct TrReader {
  int off[2];
  __device__ __forceinline__ explicit TrReader(int lane) {
    const int i = lane & 15, G = lane >> 4;
    const int rl = 4 * (G >> 1) + (i >> 2);              // row within a 16-row chunk, bits 0..2
    const int sw = tile_swz(rl);
    const int r = 2 * (G & 1) + ((i >> 1) & 1);          // chunk within a 32-column tile
    const int sub = 8 * (i & 1);                         // byte offset inside the chunk
#pragma unroll
    for (int n = 0; n < 2; ++n) off[n] = rl * (2 * D) + 64 * (n ^ (sw >> 2)) + 16 * (r ^ (sw & 3)) + sub;
  }
  // Same operand as tile_tr8<D>(t, c16, mt, lane).
  __device__ __forceinline__ bf16x8 operator()(const char *t, int c16, int mt) const {
    const char *p = t + off[mt & 1] + 128 * (mt >> 1) + 16 * c16 * (2 * D);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BD_LDS_V4I16(p));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BD_LDS_V4I16(p + 8 * (2 * D)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  }
};

// s_waitcnt with vmcnt(N) and the other counters left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) (LDS reads of this wave complete), other counters free.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }
__device__ __forceinline__ void wg_barrier() { __builtin_amdgcn_s_barrier(); }

}  // namespace bdattn
