// Kernel argument blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdattn {

struct FwdArgs {
  const void *q;            // [n_q][h_q][d] bf16
  const void *k[2];         // per key segment: [n][h_kv][d] bf16 (natural layout)
  const void *vt[2];        // per key segment: [h_kv][d][kpad] bf16, keys permuted within 16
  int64_t kpad[2];
  int32_t n_seg[2];
  void *o;                  // [n_q][h_q][d], fp32 or bf16
  float *lse;               // [h_q][n_q]
  const int32_t *rows;      // [n_q][4] row bounds
  const int32_t *items;     // [n_items][12] tile descriptors, longest first
  int32_t n_items, n_q, h_q, h_kv, group;
  int32_t o_f32;
  float scale_log2;         // softmax scale * log2(e)
};

struct BwdArgs {
  const void *q, *dout;     // [n_q][h_q][d] bf16
  const void *k[2], *v[2];  // per segment: [n][h_kv][d] bf16
  const void *kt[2];        // per segment: [h_kv][d][kpad] bf16 (natural key order)
  int64_t kpad[2];
  int32_t n_seg[2];
  const void *qt, *dot;     // prepared slabs: [n_bq][h_q][d][BWD_BM] bf16, rows permuted within 16
  const float *lse, *delta; // [h_q][n_q]
  float *dq;                // [n_q][h_q][d] fp32, accumulated
  void *dk[2], *dv[2];      // per segment: [n][h_kv][d] bf16
  const int32_t *rows;      // [n_q][4]
  const int32_t *bq;        // [n_bq][12]
  const int32_t *ktiles;    // [n_kt][4]
  const int32_t *list;      // [n_list]
  int32_t n_kt, n_bq, n_q, h_q, h_kv, group;
  float scale, scale_log2;
};

struct PrepArgs {
  const void *q, *o, *dout; // [n_q][h_q][d]; o fp32 or bf16
  int32_t o_f32;
  float *delta;             // [h_q][n_q]
  float *dq_zero;           // optional [n_q][h_q][d] fp32 accumulator to clear
  void *qt, *dot;           // [n_bq][h_q][d][BWD_BM]
  const int32_t *bq;        // [n_bq][12]
  int32_t n_bq, n_q, h_q;
};

hipError_t launch_transpose(const void *x, int64_t n, int32_t h_kv, int32_t d, int64_t kpad, bool permute,
                            void *out, hipStream_t s);
hipError_t launch_fwd(const FwdArgs &a, int32_t d, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int32_t d, hipStream_t s);
hipError_t launch_prepare(const PrepArgs &a, int32_t d, hipStream_t s);
hipError_t launch_merge(int32_t n_parts, const void *o_parts, bool parts_f32, const float *lse_parts,
                        int64_t n_rows, int32_t h, int32_t d, void *o_out, bool out_f32, float *lse_out,
                        hipStream_t s);
hipError_t launch_dq_finalize(const float *acc, void *out, int64_t n, hipStream_t s);

}  // namespace bdattn
