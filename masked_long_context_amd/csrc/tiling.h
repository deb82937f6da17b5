// Tile shapes shared by the host scheduler and the gfx950 kernels.
#pragma once

// Forward (and the query-major dQ kernel): one workgroup owns BDATTN_FWD_BM
// query rows of one q-head (32 per wave).  The forward walks the legal keys
// BDATTN_FWD_STEP at a time (two 64-row LDS tiles of K and of V per step), the
// dQ kernel BDATTN_FWD_BN at a time; every key tile loaded serves all waves.
#define BDATTN_FWD_WAVES 8
#define BDATTN_FWD_BM (32 * BDATTN_FWD_WAVES)
#define BDATTN_FWD_BN 64
#define BDATTN_FWD_STEP 128
// Backward: one workgroup owns BDATTN_BWD_BN keys of one KV head and walks the
// query tiles (BDATTN_BWD_BM rows) that attend them, for every q-head of the group.
#define BDATTN_BWD_WAVES 4
#define BDATTN_BWD_BM 64
#define BDATTN_BWD_BN 128
// Threads of a dK/dV workgroup (eight waves: four per role).
#define BDATTN_DKDV_THREADS 512
// A launch's grid may hold at most this many work-items (HIP's limit on
// gridDim.x * blockDim.x); plans whose grids would exceed it are rejected.
#define BDATTN_MAX_GRID_ITEMS 0xFFFFFFFFLL
// A plan whose dK/dV kernel would occupy few workgroups splits every key tile's
// query-tile walk over up to BDATTN_MAX_SPLIT workgroups, each writing fp32
// partial dK/dV that a reduction kernel sums in a fixed order.  Automatic
// splitting aims at BDATTN_SPLIT_TARGET workgroups, keeps at least
// BDATTN_SPLIT_MIN_ITERS query tiles per workgroup, and keeps the partials
// within BDATTN_SPLIT_MAX_BYTES.
#define BDATTN_MAX_SPLIT 8
#define BDATTN_SPLIT_TARGET 1024
#define BDATTN_SPLIT_MIN_ITERS 8
#define BDATTN_SPLIT_MAX_BYTES (512LL << 20)
// Alignment of every buffer carved out of a workspace.
#define BDATTN_ALIGN 256

#define BDATTN_IMAGE_MAGIC 0x62646174  // "bdat"
