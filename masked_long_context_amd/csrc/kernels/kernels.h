// Kernel argument blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "bdattn.h"

namespace bdattn {

// The clean key segment (segment 0) in one buffer (n = 1: k[0], v[0]) or split
// over n buffers of len rows each, the last holding the rest: row r of the
// segment is row r - i len of buffer i = min(r / len, n - 1).  len is a multiple
// of BDATTN_BWD_BN (and so of every key tile and forward step) when n > 1, so a
// tile never straddles two buffers.
struct KvShardTable {
  const void *k[BDATTN_MAX_SHARDS], *v[BDATTN_MAX_SHARDS];
  int32_t n, len;
};
// Gradient buffers of the same split (backward only).
struct GradShardTable {
  void *dk[BDATTN_MAX_SHARDS], *dv[BDATTN_MAX_SHARDS];
};

struct FwdArgs {
  const void *q;            // [n_q][h_q][d] bf16
  const void *k[2], *v[2];  // per key segment: [n][h_kv][d] bf16 (segment 0: sh.k[0], sh.v[0])
  KvShardTable sh;          // segment 0's buffers
  int32_t n_seg[2];
  void *o;                  // [n_q][h_q][d], fp32 or bf16
  float *lse;               // [h_q][n_q]
  const int32_t *rows;      // [n_q][4] row bounds
  const int32_t *items;     // [n_items][12] query tiles, longest first
  int32_t n_items, n_q, h_q, h_kv, group;
  int32_t o_f32;
  float scale_log2;         // softmax scale * log2(e)
};

struct BwdArgs {
  const void *q, *dout;     // [n_q][h_q][d] bf16
  const void *k[2], *v[2];  // per segment: [n][h_kv][d] bf16 (segment 0: sh.k[0], sh.v[0])
  KvShardTable sh;          // segment 0's buffers
  GradShardTable gsh;       // segment 0's gradient buffers, split as sh
  int32_t n_seg[2];
  const float *lse, *delta; // [h_q][n_q]
  float *dq;                // [n_q][h_q][d] fp32, accumulated
  void *dk[2], *dv[2];      // per segment: [n][h_kv][d] bf16 (segment 0: gsh.dk[0], gsh.dv[0])
  const int32_t *rows;      // [n_q][4]
  const int32_t *items;     // [n_items][12] query tiles of the dQ kernel (the forward tiling)
  const int32_t *bq;        // [n_bq][12] query tiles of the dK/dV kernel
  const int32_t *ktiles;    // [n_kt][4]
  const int32_t *list;      // [n_list]
  const int32_t *lrec;      // [n_list][4] per list entry {q0, rows, full, q-tile}
  int32_t n_items, n_kt, n_bq, n_q, h_q, h_kv, group;
  float scale, scale_log2;
  // dK/dV workgroups per key tile; above 1 each writes fp32 partials to
  // part[s] ([2][split][n_seg][h_kv][d], dK then dV) and a reduction sums them
  int32_t split;
  float *part[2];
};

struct PrepArgs {
  const void *o, *dout;     // [n_q][h_q][d]; o fp32 or bf16
  int32_t o_f32;
  float *delta;             // [h_q][n_q]
  float *dq_zero;           // optional [n_q][h_q][d] fp32 accumulator to clear
  int32_t n_q, h_q;
};

hipError_t launch_fwd(const FwdArgs &a, int32_t d, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int32_t d, hipStream_t s, bool dkdv, bool dq);
hipError_t launch_prepare(const PrepArgs &a, int32_t d, hipStream_t s);
hipError_t launch_merge(int32_t n_parts, const void *o_parts, bool parts_f32, const float *lse_parts,
                        int64_t n_rows, int32_t h, int32_t d, void *o_out, bool out_f32, float *lse_out,
                        hipStream_t s);
hipError_t launch_cast_bf16(const float *src, void *out, int64_t n, hipStream_t s);

}  // namespace bdattn
