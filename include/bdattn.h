/*
 * bdattn.h -- C ABI of the MI355X (gfx950) BDLM-masked core attention library.
 *
 * What it computes.  softmax(Q K^T) V and its gradients for ONE rank's share of
 * block-diffusion (BDLM) training under context-sharded block parallelism
 * (CSBP), against one clean K/V range per call, plus the exact log-sum-exp
 * merge of the per-range partials and a varlen entry point for packed shards.
 *
 *  - Mask: "rit.work explainer of CSBP", section on why conventional context
 *    parallelism sends extra data: each corrupted (noised) target block sees
 *    the clean prefix of the PRECEDING blocks and its own noised version;
 *    corrupted K/V serve only the block that owns them.  "Block Parallelism
 *    For Efficient Distributed Long-Context Diffusion Language Model
 *    Training", English abstract: autoregressive across blocks, parallel
 *    denoising within a block, so a clean token sees the clean tokens of its
 *    own and all earlier blocks.  Exactly:
 *        clean row at position p   -> clean key t iff t/B <= p/B
 *        clean row                 -> corrupted key: never
 *        corrupted block b (slot m)-> clean key t iff t/B <  b
 *                                  -> corrupted key iff it is in slot m
 *  - Sharding: the same abstract -- one rank owns each corrupted block, the
 *    clean sequence is sharded by position across the ranks, corrupted K/V
 *    stay local, and the training semantics are preserved; hence per-range
 *    partials (O_s, LSE_s) merge exactly and the backward of a range uses the
 *    merged LSE.
 *  - Varlen: "Efficient Long-context Language Model Training by Core
 *    Attention Disaggregation", English abstract: core attention over fused
 *    batches of token-level shards of arbitrary length.
 *
 * Conventions.  scale <= 0 selects 1/sqrt(head_dim).  LSE is the natural-log
 * sum of exp(scale * q.k) over the legal keys, fp32.  q-head h reads KV head
 * h / (h_q / h_kv).  A row with no legal key gets O = 0 and LSE = -inf.
 *
 * Layouts (all row-major, contiguous in the last dimension):
 *   Q, O, dO, dQ          [n_q][h_q][head_dim]  rows: the clean query rows,
 *                                             then B rows per owned block in
 *                                             owned_blocks order
 *   K/V clean range       [kv_clean_len][h_kv][head_dim]  (pointer = first row of the range)
 *   K/V local corrupted   [n_owned * B][h_kv][head_dim]   (same slot order as the rows)
 *   LSE, delta            [h_q][n_q] fp32
 *   packed varlen Q/O/dO  [total][h_q][head_dim], K/V [total][h_kv][head_dim]
 * Tensors are bf16 unless stated.  Device pointers must be 16-byte aligned.
 * Sizes: query rows, keys of each segment and packed rows are each below 2^30
 * (plans beyond that are rejected with BDATTN_EINVAL); the kernels form every
 * element offset in 64-bit arithmetic.  The library cannot see the extent of a
 * buffer: each must hold at least the rows the plan implies (the Python binding
 * checks every tensor's shape, dtype, device and contiguity before each call).
 *
 * Ownership.  Every device buffer, including the workspace, belongs to the
 * caller; the library never allocates device memory.
 * A plan holds host memory only (plus a pinned host copy of its tables, made
 * on first use); it is immutable and may be shared between threads.  A plan
 * must not be destroyed while work enqueued with it may still run
 * (bdattn_plan_destroy waits for the device if the plan was ever used).
 *
 * Errors.  Every entry point returns a bdattn_status; no C++ exception crosses
 * the ABI.  Arguments are validated before any HIP call (so validation runs on
 * a machine without a GPU).  HIP failures map to BDATTN_EHIP.
 * bdattn_last_error() returns a thread-local message for the last failure.
 *
 * Streams.  Every compute entry point is asynchronous on `stream` (0 = the
 * null stream) and does not synchronize.
 */
#ifndef BDATTN_H
#define BDATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BDATTN_OK = 0,
  BDATTN_EINVAL = -1,        /* null pointer, negative size, bad head counts ...            */
  BDATTN_EALIGN = -2,        /* offsets/lengths not multiples of block_size, misaligned ptr */
  BDATTN_EUNSUPPORTED = -3,  /* head_dim not in {64, 128}, dtype not supported            */
  BDATTN_EWORKSPACE = -4,    /* workspace too small                                         */
  BDATTN_EHIP = -5           /* a HIP runtime call failed                                   */
} bdattn_status;

typedef enum { BDATTN_BF16 = 0, BDATTN_F32 = 1 } bdattn_dtype;

/* Most buffers a clean K/V range may be split over (bdattn_kv_shards), and the
 * multiple of positions each buffer but the last must hold. */
#define BDATTN_MAX_SHARDS 16
#define BDATTN_SHARD_ALIGN 128

/* One rank's BDLM problem against ONE clean K/V range. */
typedef struct {
  int64_t clean_len;          /* L: whole clean sequence length, multiple of block_size       */
  int32_t block_size;         /* B >= 1                                                        */
  int64_t q_clean_offset;     /* global position of the first clean query row, multiple of B  */
  int64_t q_clean_len;        /* clean query rows (multiple of B, may be 0)                     */
  const int64_t *owned_blocks;/* HOST array of n_owned global block ids in row order; each in
                                 [0, L/B); copied by bdattn_plan_create                        */
  int64_t n_owned;
  int64_t kv_clean_offset;    /* first clean position of this call's K/V range (multiple of B)  */
  int64_t kv_clean_len;       /* length of the range (multiple of B, may be 0)                  */
  int32_t with_local_corrupt; /* 1: this call also attends the local corrupted K/V              */
  int32_t h_q, h_kv;          /* h_q % h_kv == 0                                                */
  int32_t head_dim;           /* 64 or 128                                                      */
  float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim)                                  */
} bdattn_problem;

typedef struct bdattn_plan bdattn_plan;

/* Build the host-side block-sparse tile schedule of a BDLM problem: the legal
 * (query-tile, key-tile) pairs only, each marked full (no masked pair) or
 * partial, longest tiles first.  *out receives a new plan. */
int bdattn_plan_create(const bdattn_problem *problem, bdattn_plan **out);

/* Plan for packed independent shards: cu_seqlens is a HOST int32 array of
 * n_seqs + 1 non-decreasing offsets starting at 0; shard i owns rows and keys
 * [cu[i], cu[i+1]).  causal = 1: row r sees keys cu[i] <= k <= r of its shard;
 * causal = 0: all keys of its shard. */
int bdattn_plan_create_varlen(const int32_t *cu_seqlens, int32_t n_seqs, int32_t causal,
                              int32_t h_q, int32_t h_kv, int32_t head_dim, float softmax_scale,
                              bdattn_plan **out);

/* Plan for core-attention tasks that carry their own key context ("Efficient
 * Long-context Language Model Training by Core Attention Disaggregation",
 * English abstract: core attention split into token-level tasks and rebatched
 * into fused varlen batches).  q_cu and k_cu are HOST int32 arrays of
 * n_tasks + 1 non-decreasing offsets starting at 0 (copied): task i owns query
 * rows [q_cu[i], q_cu[i+1]) of the packed Q and key rows [k_cu[i], k_cu[i+1])
 * of the packed K/V.  causal = 1 aligns the queries with the END of their
 * context (bottom-right): query j of a task with q_len rows and k_len keys sees
 * its keys 0 .. k_len - q_len + j (none when that is negative, so a task with
 * k_len < q_len has leading rows with no key: O = 0, LSE = -inf).  causal = 0:
 * every query sees all k_len keys.  Use it with the varlen compute calls,
 * passing the packed task K/V as k and v (a task's context may repeat keys of
 * another task; each copy gets its own dK/dV rows). */
int bdattn_plan_create_tasks(const int32_t *q_cu, const int32_t *k_cu, int32_t n_tasks,
                             int32_t causal, int32_t h_q, int32_t h_kv, int32_t head_dim,
                             float softmax_scale, bdattn_plan **out);

/* Split packed causal documents into core-attention tasks of bounded work
 * (same paper and passage: token-level tasks that a scheduler rebatches).
 * cu_seqlens: HOST int32, n_docs + 1 non-decreasing offsets from 0.  Each
 * document is cut into runs of consecutive rows, greedily from its first row,
 * so that a run's causal pairs (row x of the document sees its x + 1 prefix
 * keys) stay <= max_pairs_per_task; a single row above the bound forms its own
 * task.  Task t gets the run as its queries and the document prefix up to the
 * run's end as its key context, so its plan (causal = 1) reproduces causal
 * attention of the document.  Writes at most cap tasks: q_cu and k_cu
 * (cap + 1 entries, cumulative offsets into the packed task queries and task
 * contexts) and kv_src (cap entries: packed row where the task's context
 * starts, i.e. its document's first row).  Returns the number of tasks (call
 * with cap = 0 to size the arrays) or a negative bdattn_status
 * (BDATTN_EINVAL also when the summed context rows exceed 2^30). */
int64_t bdattn_cad_split(const int32_t *cu_seqlens, int32_t n_docs, int64_t max_pairs_per_task,
                         int32_t *q_cu, int32_t *k_cu, int32_t *kv_src, int64_t cap);

void bdattn_plan_destroy(bdattn_plan *plan);

/* Size (bytes) of the per-call workspace: the plan's tables, uploaded by each call,
 * and, when the plan splits its dK/dV key tiles, the fp32 dK/dV partials. */
int64_t bdattn_plan_workspace_bytes(const bdattn_plan *plan);

/* Keeps the plan's tables in `workspace` (>= bdattn_plan_workspace_bytes, 256-byte
 * aligned): copies them there once, on `stream`, and every later compute call
 * given this plan and this same workspace skips its own upload (a host-to-device
 * copy that the call's kernels would wait for).  For a plan run many times, such
 * as one rank's shard in every training step.  Calls with another workspace
 * upload as before.  A plan keeps at most one workspace (a new call replaces the
 * previous one), and a workspace holds one plan's tables: an upload of another
 * plan's tables over any of those bytes (any call, or this one) ends the first
 * plan's claim.
 * workspace NULL: ends this plan's claim.  The library cannot see other writes:
 * while the tables are kept the caller must not write the workspace (other than
 * through this plan's calls) nor free it; end the claim first (or destroy the
 * plan).  Errors: EINVAL (plan NULL), EALIGN, EWORKSPACE, EHIP. */
int bdattn_plan_keep_tables(bdattn_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);

/* Workgroups per key tile of the dK/dV kernel (a schedule choice; results do not
 * depend on it beyond fp32 rounding order, and are deterministic for each value).
 * With one, each workgroup walks every query tile that attends its 128 keys and
 * writes dK/dV directly.  A problem with few key tiles would leave most compute
 * units idle that way, so a plan splits each walk over `split` workgroups that
 * write fp32 partials into the workspace, summed in a fixed order by a reduction
 * kernel.  plan_create picks the split automatically (0); this call overrides it
 * (0 = automatic, 1..8 = fixed) and must come before the plan's first use
 * (BDATTN_EINVAL otherwise, and for values outside 0..8).  It changes the
 * workspace size.  bdattn_plan_dkdv_split returns the value in force. */
int bdattn_plan_set_dkdv_split(bdattn_plan *plan, int32_t split);
int32_t bdattn_plan_dkdv_split(const bdattn_plan *plan);
/* Head counts and head dim of the plan's problem. */
int bdattn_plan_heads(const bdattn_plan *plan, int32_t *h_q, int32_t *h_kv, int32_t *head_dim);
/* Legal (query, key) pairs per query head: the useful-work count. */
int64_t bdattn_plan_useful_pairs(const bdattn_plan *plan);
/* Query rows, and key rows of the clean (or packed) range and of the local corrupted K/V. */
int64_t bdattn_plan_n_q(const bdattn_plan *plan);
int64_t bdattn_plan_n_kv(const bdattn_plan *plan, int32_t segment /* 0 clean/packed, 1 corrupted */);

/* Introspection of the schedule (for tests).  which:
 *   0 row bounds : int32[n_q][4]  = {lo_a, hi_a, lo_b, hi_b}; row r may attend keys
 *                  [lo_a, hi_a) of segment 0 and [lo_b, hi_b) of segment 1
 *   1 fwd items  : int32[n][12]   = {q0, rows, seg0 lo_min, lo_max, hi_min, hi_max,
 *                                    seg1 lo_min, lo_max, hi_min, hi_max, cost, 0}
 *   2 bwd q-tiles: int32[n][12]   (same layout, backward query tiling)
 *   3 bwd k-tiles: int32[n][4]    = {segment, k0, list_begin, list_end}
 *   4 bwd list   : int32[n]       = q-tile index | (full << 31)
 * Returns the number of records, or a negative status; copies at most `cap`
 * records into `out` when out != NULL. */
int64_t bdattn_plan_export(const bdattn_plan *plan, int32_t which, int32_t *out, int64_t cap);

/* Forward partial of one clean K/V range (+ the local corrupted K/V when the
 * plan's problem has with_local_corrupt).
 * Source: "Block Parallelism For Efficient Distributed Long-Context Diffusion
 * Language Model Training", English abstract (the clean sequence is sharded by
 * position, so a rank meets the clean K/V one range at a time; one rank owns
 * each corrupted block), and the rit.work explainer of CSBP, section on why
 * conventional context parallelism sends extra data (the mask above: clean
 * prefix of the preceding blocks plus the block's own noised version).  The
 * partial carries its log-sum-exp so that ranges merge exactly.
 * Computes, for every row r and q-head h over the legal keys j of this range:
 *   LSE[h][r] = ln sum_j exp(scale q_r.k_j),  O[r][h] = sum_j exp(scale q_r.k_j - LSE) v_j
 * (a row with no legal key in the range: O = 0, LSE = -inf).
 * Writes O ([n_q][h_q][d], o_dtype BDATTN_F32 or BDATTN_BF16) and LSE
 * ([h_q][n_q] fp32) with `=`.  q: [n_q][h_q][d]; k_clean/v_clean:
 * [kv_clean_len][h_kv][d] (the range's first row); k_corr/v_corr: [n_owned*B][h_kv][d],
 * may be NULL when the plan has no local corrupted keys.
 * workspace: >= bdattn_plan_workspace_bytes, 256-byte aligned; each call
 * uploads the plan's tables into it on `stream`, so calls that may overlap
 * need separate workspaces.  Errors: EINVAL (NULL pointer, varlen plan),
 * EALIGN (misaligned pointer), EUNSUPPORTED (o_dtype), EWORKSPACE, EHIP. */
int bdattn_fwd(const bdattn_plan *plan, const void *q, const void *k_clean, const void *v_clean,
               const void *k_corr, const void *v_corr, void *o, int32_t o_dtype, float *lse,
               void *workspace, int64_t workspace_bytes, void *stream);

/* bdattn_fwd for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments and
 * results as bdattn_fwd (BDLM plans), without the workspace: the plan's
 * forward tables are copied into a static device array of 8 MiB that the
 * library holds on each GPU it runs on until the process ends, so the call
 * allocates nothing (no hipMalloc, no pinned copy; the tables are copied from
 * the plan's host memory on `stream`).  Limit: the forward tables (16 bytes per
 * query row plus 48 per 256-row tile, about 500K query rows) must fit in
 * 8 MiB, else BDATTN_EWORKSPACE before any HIP call.  Every call on a GPU
 * shares that GPU's array, which keeps the last call's tables: calls that may
 * overlap on one GPU (other streams, other threads) race on it and must be
 * ordered by the caller.  The device is the current one; the stream must
 * belong to it. */
int bdattn_fwd_static(const bdattn_plan *plan, const void *q, const void *k_clean, const void *v_clean,
                      const void *k_corr, const void *v_corr, void *o, int32_t o_dtype, float *lse,
                      void *stream);

/* Exact merge of n_parts partials over disjoint key sets.
 * Source: the block-parallelism abstract (CSBP preserves the BDLM training
 * semantics) and the rit.work explainer's opening paragraph (the loss and the
 * gradients do not change): the per-range partials must combine into exactly
 * the unsharded attention, which the log-sum-exp identity gives:
 *   m = max_s LSE_s;  LSE = m + ln sum_s exp(LSE_s - m);  O = sum_s exp(LSE_s - LSE) O_s
 * (all partials -inf -> O = 0, LSE = -inf).  o_parts: [n_parts][n_rows][h][d] in
 * part_dtype, lse_parts: [n_parts][h][n_rows] fp32; o_out [n_rows][h][d] in out_dtype,
 * lse_out [h][n_rows] fp32.  d in {64, 128}.  For a training step keep
 * out_dtype BDATTN_F32 and round with bdattn_cast_f32_bf16: the backward's
 * delta is then taken from the unrounded output.  Errors: EINVAL (n_parts < 1,
 * NULL pointer), EALIGN, EUNSUPPORTED (d, dtype), EHIP. */
int bdattn_lse_merge(int32_t n_parts, const void *o_parts, int32_t part_dtype, const float *lse_parts,
                     int64_t n_rows, int32_t h, int32_t d, void *o_out, int32_t out_dtype,
                     float *lse_out, void *stream);

/* Backward preparation, once per rank step (shared by every K/V range):
 * delta[h][r] = sum_d dO[r][h][d] * O[r][h][d] (fp32 [h_q][n_q]) from the MERGED
 * output O (o_dtype; pass the fp32 merged output where it is kept: with one
 * dominant key dS = P o (dP - delta) is a small difference, and the bf16
 * rounding of O alone moves it), and, when dq_accum is not NULL, dq_accum
 * (fp32 [n_q][h_q][d]) cleared to 0.  Only the plan's query side (n_q, h_q,
 * head_dim) is used.  Errors: EINVAL, EALIGN, EUNSUPPORTED (o_dtype), EHIP. */
int bdattn_bwd_prepare(const bdattn_plan *plan, const void *o, int32_t o_dtype, const void *dout,
                       float *delta, float *dq_accum, void *stream);

/* Backward of one K/V range given the MERGED lse and the prepared delta.
 * Source: the rit.work explainer of CSBP, section on why conventional context
 * parallelism sends extra data (CSBP returns only the gradients of the clean
 * K/V to their owners; the corrupted K/V gradients stay with their block), and
 * the block-parallelism abstract (training semantics preserved: with the merged
 * LSE the probabilities of a range are exact, so per-range backwards add up to
 * the unsharded one).
 * Signature.  Delta is not computed here: bdattn_bwd_prepare computes it once
 * per rank step from the merged output and every range's call reads it, so
 * this call takes no O and no "delta ready" flag (it never writes delta).
 * Computes:
 *   P = exp(scale Q K^T - LSE) on the legal pairs, dS = P o (dO V^T - delta)
 *   dq_accum += scale dS K    (fp32 [n_q][h_q][d]; each call adds its range)
 *   dk = scale dS^T Q, dv = P^T dO, summed over the q-heads of each KV head and
 *   written with `=` (bf16) for every key of the range (zeros for keys no query
 *   attends).
 * Two kernels run in order on `stream`: a key-major one for dK/dV and a
 * query-major one for dQ.  dk_corr/dv_corr may be NULL when the plan has no
 * local corrupted keys.  workspace: >= bdattn_plan_workspace_bytes.
 * Errors: EINVAL (NULL pointer, varlen plan), EALIGN, EWORKSPACE, EHIP. */
int bdattn_bwd(const bdattn_plan *plan, const void *q, const void *k_clean, const void *v_clean,
               const void *k_corr, const void *v_corr, const void *dout, const float *lse,
               const float *delta, float *dq_accum, void *dk_clean, void *dv_clean, void *dk_corr,
               void *dv_corr, void *workspace, int64_t workspace_bytes, void *stream);

/* The two steps of bdattn_bwd as separate calls (same kernels, same launch
 * configuration), for callers that schedule or time them apart:
 * bdattn_bwd_dkdv writes dK/dV of the range (key-major kernel);
 * bdattn_bwd_dq adds the range's contribution to dq_accum (query-major kernel).
 * Either works on a BDLM or a varlen plan (varlen: pass the packed K/V as the
 * clean range and NULL for the corrupted pointers). */
int bdattn_bwd_dkdv(const bdattn_plan *plan, const void *q, const void *k_clean, const void *v_clean,
                    const void *k_corr, const void *v_corr, const void *dout, const float *lse,
                    const float *delta, void *dk_clean, void *dv_clean, void *dk_corr, void *dv_corr,
                    void *workspace, int64_t workspace_bytes, void *stream);
int bdattn_bwd_dq(const bdattn_plan *plan, const void *q, const void *k_clean, const void *v_clean,
                  const void *k_corr, const void *v_corr, const void *dout, const float *lse,
                  const float *delta, float *dq_accum, void *workspace, int64_t workspace_bytes,
                  void *stream);

/* Every resident clean shard in one launch per kernel.
 * Source: the block-parallelism abstract (the clean sequence is sharded by
 * position, and a rank attends the clean K/V of the blocks before its own) and
 * the rit.work explainer of CSBP, section on why conventional context
 * parallelism sends extra data (what a rank receives is clean K/V).  When the
 * shards a rank attends are all resident, each in the buffer it arrived in,
 * per-range partials and their merge are not needed: one online-softmax pass
 * over all of them merges them exactly in registers (the log-sum-exp identity
 * of bdattn_lse_merge, applied key tile by key tile), and no fp32 partial
 * leaves the chip.
 * The plan covers the whole range of the shards (kv_clean_offset: the first
 * shard's first position; kv_clean_len: the sum of their lengths).  Buffer i
 * holds positions [i shard_len, (i + 1) shard_len) of that range, the last one
 * the rest: 1 <= n_shards <= BDATTN_MAX_SHARDS; for n_shards > 1, shard_len is a
 * multiple of BDATTN_SHARD_ALIGN and every buffer holds at least one position,
 * (n_shards - 1) shard_len < kv_clean_len <= n_shards shard_len (n_shards = 1:
 * shard_len is ignored).  k[i], v[i]: [len_i][h_kv][head_dim] bf16, len_i the
 * buffer's positions; dk[i], dv[i] (backward only, else ignored): the same
 * shapes, written with `=`, zeros for keys no query attends.  The struct is
 * read on the host during the call.  Any plan (a varlen plan: its packed K/V
 * split the same way, NULL corrupted pointers).
 * Results are bit for bit those of bdattn_fwd / bdattn_bwd (or the varlen
 * calls) with the range in one buffer.  Errors: as bdattn_fwd / bdattn_bwd;
 * EINVAL also for kv NULL, n_shards out of range, or buffers that do not cover
 * the range as above; EALIGN for shard_len not a multiple of BDATTN_SHARD_ALIGN. */
typedef struct bdattn_kv_shards {
  int32_t n_shards;
  int64_t shard_len;
  const void *k[BDATTN_MAX_SHARDS];
  const void *v[BDATTN_MAX_SHARDS];
  void *dk[BDATTN_MAX_SHARDS];
  void *dv[BDATTN_MAX_SHARDS];
} bdattn_kv_shards;

int bdattn_fwd_shards(const bdattn_plan *plan, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                      const void *v_corr, void *o, int32_t o_dtype, float *lse, void *workspace,
                      int64_t workspace_bytes, void *stream);
int bdattn_bwd_shards(const bdattn_plan *plan, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                      const void *v_corr, const void *dout, const float *lse, const float *delta,
                      float *dq_accum, void *dk_corr, void *dv_corr, void *workspace, int64_t workspace_bytes,
                      void *stream);
int bdattn_bwd_dkdv_shards(const bdattn_plan *plan, const void *q, const bdattn_kv_shards *kv,
                           const void *k_corr, const void *v_corr, const void *dout, const float *lse,
                           const float *delta, void *dk_corr, void *dv_corr, void *workspace,
                           int64_t workspace_bytes, void *stream);
int bdattn_bwd_dq_shards(const bdattn_plan *plan, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                         const void *v_corr, const void *dout, const float *lse, const float *delta,
                         float *dq_accum, void *workspace, int64_t workspace_bytes, void *stream);

/* dq (bf16) = dq_accum (fp32), n_elems elements (round to nearest even). */
int bdattn_dq_finalize(const float *dq_accum, void *dq, int64_t n_elems, void *stream);

/* dst (bf16) = src (fp32), n_elems elements, round to nearest even: the bf16
 * layer output from the fp32 merged output kept for the backward. */
int bdattn_cast_f32_bf16(const float *src, void *dst, int64_t n_elems, void *stream);

/* Varlen packed shards: the same kernels over a plan from bdattn_plan_create_varlen
 * or bdattn_plan_create_tasks (k and v: [n_keys][h_kv][head_dim], n_keys =
 * cu_seqlens[n_seqs] or k_cu[n_tasks]; dk and dv have the same shape). */
int bdattn_varlen_fwd(const bdattn_plan *plan, const void *q, const void *k, const void *v, void *o,
                      int32_t o_dtype, float *lse, void *workspace, int64_t workspace_bytes,
                      void *stream);
int bdattn_varlen_bwd(const bdattn_plan *plan, const void *q, const void *k, const void *v,
                      const void *dout, const float *lse, const float *delta, float *dq_accum,
                      void *dk, void *dv, void *workspace, int64_t workspace_bytes, void *stream);

/* Thread-local message describing the last non-OK status on this thread. */
const char *bdattn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BDATTN_H */
