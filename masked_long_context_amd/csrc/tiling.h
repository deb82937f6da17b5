// Tile shapes shared by the host scheduler and the gfx950 kernels.
#pragma once

// Forward (and the query-major dQ kernel): one workgroup owns BDATTN_FWD_BM
// query rows of one q-head (32 per wave) and walks the legal keys BDATTN_FWD_BN
// at a time; every key tile it loads serves all its waves.
#define BDATTN_FWD_WAVES 8
#define BDATTN_FWD_BM (32 * BDATTN_FWD_WAVES)
#define BDATTN_FWD_BN 64
// Backward: one workgroup owns BDATTN_BWD_BN keys of one KV head and walks the
// query tiles (BDATTN_BWD_BM rows) that attend them, for every q-head of the group.
#define BDATTN_BWD_WAVES 4
#define BDATTN_BWD_BM 64
#define BDATTN_BWD_BN 128
// Alignment of every buffer carved out of a workspace.
#define BDATTN_ALIGN 256

#define BDATTN_IMAGE_MAGIC 0x62646174  // "bdat"
