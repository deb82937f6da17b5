// LDS tiles for the gfx950 attention kernels.
//
// A tile is 64 rows of a row-major bf16 matrix with D elements per row, copied
// from global memory straight into LDS by buffer_load_dwordx4 ... lds (each
// lane of a wave moves 16 bytes; a wave-wide load fills 1 KB of LDS in lane order),
// in the swizzled chunk layout of lds_layout.h, and read back as MFMA operands
// with one of two fixed lane patterns whose per-lane offsets are computed once.
#pragma once
#include "common.h"
#include "lds_layout.h"

namespace bdattn {

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define BD_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define BD_LDS_V4I16(p) ((__attribute__((address_space(3))) v4i16 *)(p))

template <int D>
using Tile = TileShape<D>;

// Word 3 of a raw buffer resource on gfx9 (CDNA): 32-bit data format, no
// swizzle, no index stride; offsets past num_records read as zero.
constexpr int kBufferWord3 = 0x00020000;

// This wave's share of the asynchronous copy of 64 rows starting at `g` (a
// wave-uniform pointer; row stride `stride` elements, 64 * stride < 2^30).  Rows
// at or beyond `nvalid` re-read row nvalid - 1 (the caller masks them);
// nvalid >= 1.  `wave` must be wave-uniform.  Issues Tile<D>::LOADS / NW loads.
template <int D, int NW>
__device__ __forceinline__ void tile_load(char *lds, const bf16 *g, int stride, int nvalid, int wave, int lane) {
  constexpr int PER = Tile<D>::LOADS / NW;
  static_assert(Tile<D>::LOADS % NW == 0, "tile loads must split evenly over the waves");
  // A raw buffer resource over the rows the tile may touch.  The buffer form of
  // the LDS DMA (unlike the global form) leaves the compiler's LDS read
  // counter in order, so the operand reads that follow keep exact waits.
  const int nrec = (nvalid < Tile<D>::ROWS ? nvalid : Tile<D>::ROWS) * stride * 2;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16 *>(g), (short)0, nrec, kBufferWord3);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int kb = wave * PER + i;
    int row, c;
    tile_load_src<D>(kb, lane, &row, &c);
    const int rr = row < nvalid ? row : nvalid - 1;
    const int off = (rr * stride + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, BD_LDS(lds + kb * 1024), 16, off, 0, 0, 0);
  }
}

// One dword per lane, from byte offset `off` of [base, base + bytes), into LDS at
// lds + 4 * lane (the buffer form of the LDS DMA, for the reason above).
__device__ __forceinline__ void dword_load_lds(const void *base, int bytes, int off, void *lds) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, BD_LDS(lds), 4, off, 0, 0, 0);
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Row reads: the MFMA operand for tile rows 32 tb + lane % 32, head-dim
// elements 16 c + 8 (lane / 32) .. +7 (A or B of a 32x32x16 MFMA contracting
// over the head dim).  One per-lane offset per c; tb is an immediate.
template <int D>
struct RowReader {
  int off[Tile<D>::NC];
  __device__ __forceinline__ explicit RowReader(int lane) { row_read_offsets<D>(lane, off); }
  __device__ __forceinline__ bf16x8 operator()(const char *t, int tb, int c) const {
    return *reinterpret_cast<const bf16x8 *>(t + off[c] + tb * 32 * Tile<D>::ROWB);
  }
};

// Transpose reads: for a tile X[k][m], the MFMA operand whose lane row/column is
// m = 32 mt + lane % 32 and whose 8 k-values are the rows of 16-chunk c16 in the
// order the C registers of a previous MFMA hold them (rows 16 c16 + 4 g + 0..3,
// then 16 c16 + 8 + 4 g + 0..3, g = lane / 32).  One per-lane offset per mt.
template <int D>
struct TrReader {
  int off[Tile<D>::ND];
  __device__ __forceinline__ explicit TrReader(int lane) { tr_read_offsets<D>(lane, off); }
  __device__ __forceinline__ bf16x8 operator()(const char *t, int c16, int mt) const {
    const char *p = t + 16 * c16 * Tile<D>::ROWB;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(BD_LDS_V4I16(p + off[mt]));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        BD_LDS_V4I16(p + off[mt ^ Tile<D>::TR_BX] + 8 * Tile<D>::ROWB));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
  }
};

// Orders the current scheduling region so that its LDS reads run ahead of the
// MFMAs that consume them: AHEAD operands are read first, then each MFMA is
// followed by the reads of the operand AHEAD positions later.  N MFMAs, each
// consuming one operand of READS LDS reads.  Without it the scheduler, short of
// registers, reads each operand just before its MFMA and waits for it there.
template <int N, int READS, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  static_assert(AHEAD <= N, "lookahead longer than the sequence");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * READS, 0);
#pragma unroll
  for (int k = 0; k < N - AHEAD; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

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
