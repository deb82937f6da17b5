// Tile shapes shared by the host scheduler and the gfx950 kernels.
#pragma once

// Forward: one workgroup owns BDATTN_FWD_BM query rows of one q-head and walks
// the legal keys BDATTN_FWD_BN at a time.
#define BDATTN_FWD_WAVES 4
#define BDATTN_FWD_BM 128
#define BDATTN_FWD_BN 64
// Backward: one workgroup owns BDATTN_BWD_BN keys of one KV head and walks the
// query tiles (BDATTN_BWD_BM rows) that attend them, for every q-head of the group.
#define BDATTN_BWD_WAVES 4
#define BDATTN_BWD_BM 64
#define BDATTN_BWD_BN 128
// Transposed K/V copies are padded to a multiple of this many keys.
#define BDATTN_KPAD 128
// Alignment of every buffer carved out of a workspace.
#define BDATTN_ALIGN 256

#define BDATTN_IMAGE_MAGIC 0x62646174  // "bdat"
