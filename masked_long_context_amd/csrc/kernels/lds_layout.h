// Layout of a K/V/Q/dO tile in LDS and the per-lane offsets of the reads the
// gfx950 kernels make from it.  Plain integer arithmetic, usable on the host
// (tests check it there) and on the device.
//
// A tile is 64 rows of a row-major bf16 matrix with D elements per row (2D
// bytes), cut into 16-byte chunks.  Chunk c of row r is stored at chunk position
// c ^ swz(r) of that row.  The swizzle is chosen for the gfx950 LDS, which has
// 64 four-byte banks: a ds_read_b128 is served 16 lanes (256 bytes) at a time,
// and the 16 lanes of a group must hit 16 distinct 16-byte bank groups to run at
// full rate.  Two read patterns occur:
//   * row reads (MFMA operand along the head dim, ds_read_b128): lanes 0..15 of
//     a group read the same chunk of 16 consecutive rows;
//   * transpose reads (MFMA operand down a column, ds_read_b64_tr_b16): 32 lanes
//     read 4 chunks (two 8-byte halves each) of 4 consecutive rows.
// D = 128 (16 chunks per row, every row starts on bank 0):
//   swz(r) = 4 ((r ^ (r >> 2)) mod 4) + (r mod 4)
//   a bijection on r mod 16 (row reads), whose top two bits differ across any 4
//   consecutive rows (transpose reads); moving 8 rows down flips only bit 3.
// D = 64 (8 chunks per row, two rows per 256 bytes):
//   swz(r) = 4 (((r >> 1) ^ (r >> 3)) mod 2) + ((r >> 1) mod 4)
//   a bijection on (r >> 1) mod 8 (rows of equal parity share a bank half),
//   whose bit 2 differs between rows r and r + 2; 8 rows down flips only bit 2.
#pragma once

#ifdef __HIPCC__
#define BD_HD __host__ __device__ __forceinline__
#else
#define BD_HD inline
#endif

namespace bdattn {

template <int D>
struct TileShape {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int ROWS = 64;
  static constexpr int ROWB = 2 * D;            // bytes per row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int RPK = 1024 / ROWB;       // rows per wave-wide 1 KB load
  static constexpr int LOADS = BYTES / 1024;    // wave-wide loads per tile
  static constexpr int NC = D / 16;             // 16-wide k-chunks of a head-dim contraction
  static constexpr int ND = D / 32;             // 32-wide column tiles of a transpose read
  // the transpose read's second half (8 rows further) uses column tile mt ^ TR_BX
  static constexpr int TR_BX = D == 128 ? 2 : 1;
};

template <int D>
BD_HD int tile_swz(int r) {
  if (D == 128) return (((r ^ (r >> 2)) & 3) << 2) | (r & 3);
  return ((((r >> 1) ^ (r >> 3)) & 1) << 2) | ((r >> 1) & 3);
}

// Byte offset of chunk `chunk` (0 .. CPR-1) of row `row` in the tile.
template <int D>
BD_HD int tile_off(int row, int chunk) {
  return row * TileShape<D>::ROWB + ((chunk ^ tile_swz<D>(row)) << 4);
}

// Wave-wide direct load number kb (1 KB of LDS, lane L -> bytes 16L .. 16L+15):
// the tile row and the logical chunk that lane `lane` fetches from global memory.
template <int D>
BD_HD void tile_load_src(int kb, int lane, int *row, int *chunk) {
  *row = kb * TileShape<D>::RPK + lane / TileShape<D>::CPR;
  *chunk = (lane % TileShape<D>::CPR) ^ tile_swz<D>(*row);
}

// Row reads.  The MFMA operand for rows 32 tb + (lane % 32), head-dim elements
// 16 c + 8 (lane / 32) .. +7 is at  off[c] + tb * 32 * ROWB  (NC offsets).
template <int D>
BD_HD void row_read_offsets(int lane, int *off) {
  const int j = lane & 31, g = lane >> 5, s = tile_swz<D>(j);
  for (int c = 0; c < TileShape<D>::NC; ++c) off[c] = j * TileShape<D>::ROWB + 16 * ((2 * c + g) ^ s);
}

// Transpose reads of X[k][m] (tile rows k, columns m).  In each 16-lane group,
// lane i addresses 4 elements of row i / 4 (columns 4 (i mod 4) .. +3) of a 4 x 16
// block and receives column i of it; lane group G = lane / 16 takes column half
// G mod 2 and row quad G / 2.  For a 16-row chunk c16 and column tile mt the
// first read covers rows 16 c16 + 4 (G / 2) + 0..3 (the 4 k-values rows
// 4 g .. 4 g + 3 of a C-register block), the second the same 8 rows further:
//   first:  off[mt]         + 16 c16 ROWB
//   second: off[mt ^ TR_BX] + 16 c16 ROWB + 8 ROWB          (ND offsets)
// Element (row, col) of the pattern sits at tile_off(row, col / 8) + 2 (col mod 8).
template <int D>
BD_HD void tr_read_lane(int lane, int *row_in_chunk, int *col_in_tile) {
  const int i = lane & 15, G = lane >> 4;
  *row_in_chunk = 4 * (G >> 1) + (i >> 2);
  *col_in_tile = 16 * (G & 1) + 4 * (i & 3);
}

template <int D>
BD_HD void tr_read_offsets(int lane, int *off) {
  int rl, col;
  tr_read_lane<D>(lane, &rl, &col);
  for (int m = 0; m < TileShape<D>::ND; ++m) {
    const int cc = 32 * m + col;
    off[m] = tile_off<D>(rl, cc >> 3) + 2 * (cc & 7);
  }
}

}  // namespace bdattn
