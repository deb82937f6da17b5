// Host-side block-sparse tile schedule (internal; host C++17 only).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "tiling.h"

namespace bdattn {

// Per query tile: rows [q0, q0 + rows) and, for each key segment, the bounding
// values of the rows' legal ranges [lo, hi):
//   lo_min/hi_max bound the keys any row attends (non-empty rows only);
//   lo_max/hi_min tell which key tiles need no mask: [k0, k1) is full for the
//   tile iff lo_max <= k0 and k1 <= hi_min (an empty row forces hi_min = 0).
struct SegSummary { int32_t lo_min, lo_max, hi_min, hi_max; };
struct TileDesc { int32_t q0, rows; SegSummary seg[2]; int32_t cost, pad; };
struct KTile { int32_t seg, k0, begin, end; };
static_assert(sizeof(TileDesc) == 48, "TileDesc layout");
static_assert(sizeof(KTile) == 16, "KTile layout");

struct ImageHeader {
  int32_t magic, n_q, n_fwd, n_bq, n_kt, n_list, n_seg0, n_seg1;
  int64_t off_rows, off_fwd, off_bq, off_kt, off_list, off_lrec, image_bytes;
};

struct Plan {
  uint64_t id = 0;
  int kind = 0;                 // 0: BDLM rank share, 1: varlen packed shards
  int32_t h_q = 0, h_kv = 0, d = 0;
  float scale = 0.f;
  int64_t n_q = 0;
  int64_t n_seg[2] = {0, 0};    // keys of segment 0 (clean range / packed) and 1 (local corrupted)
  std::vector<int32_t> rows;    // 4 per row: lo0, hi0, lo1, hi1
  std::vector<TileDesc> fwd;    // forward items, longest first
  std::vector<TileDesc> bq;     // backward query tiles (natural order)
  std::vector<KTile> kt;        // backward key tiles, longest list first
  std::vector<int32_t> list;    // q-tile index | full << 31, grouped per key tile
  // Per list entry {q0, rows, full, q-tile index}: the q-tile fields copied, so
  // that a key-major kernel needs one scalar load per entry.
  std::vector<int32_t> lrec;
  int64_t useful_pairs = 0;
  // Device image of the tables (uploaded into the head of each workspace).
  std::vector<uint8_t> image;
  ImageHeader hdr{};
  // Workspace = the uploaded tables, then (when the dK/dV key tiles are split)
  // the fp32 dK/dV partials of each key segment: [2][split][n_seg][h_kv][d].
  int64_t ws_bytes = 0;
  int32_t dkdv_split = 1;       // workgroups per key tile in the dK/dV kernel
  int64_t off_part[2] = {0, 0};
  // Pinned copy of `image` for asynchronous uploads (made on first use).
  void *pinned = nullptr;
  bool used = false;
};

// Both return an empty string on success, else the reason for rejecting the input.
std::string build_bdlm(Plan &p, int64_t clean_len, int32_t B, int64_t q_off, int64_t q_len,
                       const int64_t *owned, int64_t n_owned, int64_t kv_off, int64_t kv_len,
                       bool local, int32_t h_q, int32_t h_kv, int32_t d, float scale);
std::string build_varlen(Plan &p, const int32_t *cu, int32_t n_seqs, bool causal, int32_t h_q,
                         int32_t h_kv, int32_t d, float scale);
std::string build_tasks(Plan &p, const int32_t *q_cu, const int32_t *k_cu, int32_t n, bool causal, int32_t h_q,
                        int32_t h_kv, int32_t d, float scale);
// Core-attention tasks with prefix context from packed documents; returns the task
// count and the summed context rows (writes at most cap tasks: q_cu / k_cu hold
// cap + 1 entries, kv_src cap).
int64_t cad_split(const int32_t *cu, int32_t n_docs, int64_t max_pairs, int32_t *q_cu, int32_t *k_cu,
                  int32_t *kv_src, int64_t cap, int64_t *total_ctx);

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Sets the dK/dV split factor (0: automatic, else 1 .. BDATTN_MAX_SPLIT) and the
// workspace layout that follows from it.
void set_dkdv_split(Plan &p, int32_t split);
// Largest number of work-items any kernel's grid would hold on this plan.
int64_t max_grid_items(const Plan &p, int32_t split);

}  // namespace bdattn
