// C ABI of the library: argument validation (before any HIP call), status
// codes, thread-local error text, table uploads and kernel launches.
#include "bdattn.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "kernels/kernels.h"
#include "plan.h"

#include "capi_internal.h"

namespace {

thread_local std::string g_err;

}  // namespace

namespace bdattn {
namespace abi {

int fail(int code, const std::string &msg) {
  g_err = msg;
  return code;
}

}  // namespace abi
}  // namespace bdattn

namespace {

using bdattn::abi::fail;

int fail_build(const std::string &e) {
  if (e.rfind("ALIGN:", 0) == 0) return fail(BDATTN_EALIGN, e.substr(6));
  if (e.rfind("UNSUP:", 0) == 0) return fail(BDATTN_EUNSUPPORTED, e.substr(6));
  return fail(BDATTN_EINVAL, e);
}

int hip_fail(hipError_t e, const char *what) {
  return fail(BDATTN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

#define CHECK(cond, code, msg) \
  do {                         \
    if (!(cond)) return fail(code, msg); \
  } while (0)

#define HIP_CHECK(expr, what)                    \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

int check_ptr(const void *p, const char *name, bool needed) {
  if (!needed) return BDATTN_OK;
  if (!p) return fail(BDATTN_EINVAL, std::string(name) + " is NULL");
  if (!aligned(p, 16)) return fail(BDATTN_EALIGN, std::string(name) + " is not 16-byte aligned");
  return BDATTN_OK;
}

#define CHECK_PTR(p, needed)                          \
  do {                                                \
    int rc_ = check_ptr((p), #p, (needed));           \
    if (rc_ != BDATTN_OK) return rc_;                 \
  } while (0)

int check_ws(const bdattn::Plan &p, const void *ws, int64_t bytes) {
  if (!ws) return fail(BDATTN_EINVAL, "workspace is NULL");
  if (!aligned(ws, BDATTN_ALIGN)) return fail(BDATTN_EALIGN, "workspace is not 256-byte aligned");
  if (bytes < p.ws_bytes)
    return fail(BDATTN_EWORKSPACE, "workspace too small: need " + std::to_string(p.ws_bytes) + " bytes");
  return BDATTN_OK;
}

bdattn_kv_shards one_buffer(const void *k, const void *v, void *dk = nullptr, void *dv = nullptr) {
  bdattn_kv_shards kv{};
  kv.n_shards = 1;
  kv.k[0] = k;
  kv.v[0] = v;
  kv.dk[0] = dk;
  kv.dv[0] = dv;
  return kv;
}

// The clean segment's buffers against the plan: count, split and pointers (K/V
// when the segment has keys, dK/dV too when `grads`).
int check_shards(const bdattn::Plan &p, const bdattn_kv_shards *kv, bool grads) {
  if (!kv) return fail(BDATTN_EINVAL, "kv shards is NULL");
  const int n = kv->n_shards;
  if (n < 1 || n > BDATTN_MAX_SHARDS) return fail(BDATTN_EINVAL, "n_shards must be in 1 .. BDATTN_MAX_SHARDS");
  const int64_t n0 = p.n_seg[0];
  if (n > 1) {
    if (kv->shard_len <= 0 || kv->shard_len % BDATTN_SHARD_ALIGN != 0)
      return fail(BDATTN_EALIGN, "shard_len must be a positive multiple of BDATTN_SHARD_ALIGN");
    // shard_len < n0 < 2^31 first, so that the products below cannot overflow
    if (!(kv->shard_len < n0 && (n - 1) * kv->shard_len < n0 && n0 <= n * kv->shard_len))
      return fail(BDATTN_EINVAL, "the shard buffers must cover the plan's clean range, each holding at least one "
                                 "position: (n_shards - 1) shard_len < kv_clean_len <= n_shards shard_len");
  }
  for (int i = 0; i < n; ++i) {
    const std::string ix = "[" + std::to_string(i) + "]";
    int rc = check_ptr(kv->k[i], ("kv.k" + ix).c_str(), n0 > 0);
    if (rc == BDATTN_OK) rc = check_ptr(kv->v[i], ("kv.v" + ix).c_str(), n0 > 0);
    if (rc == BDATTN_OK) rc = check_ptr(kv->dk[i], ("kv.dk" + ix).c_str(), n0 > 0 && grads);
    if (rc == BDATTN_OK) rc = check_ptr(kv->dv[i], ("kv.dv" + ix).c_str(), n0 > 0 && grads);
    if (rc != BDATTN_OK) return rc;
  }
  return BDATTN_OK;
}

void fill_shards(const bdattn_kv_shards &kv, bdattn::KvShardTable &t, bdattn::GradShardTable *g) {
  t = bdattn::KvShardTable{};
  t.n = kv.n_shards;
  t.len = kv.n_shards > 1 ? (int32_t)kv.shard_len : 0;
  for (int i = 0; i < kv.n_shards; ++i) {
    t.k[i] = kv.k[i];
    t.v[i] = kv.v[i];
    if (g) {
      g->dk[i] = kv.dk[i];
      g->dv[i] = kv.dv[i];
    }
  }
}

// Workspaces that hold a kept plan's tables, and the plan: an upload by any plan
// that overlaps the bytes of another plan's kept tables ends that plan's claim.
std::mutex g_kept_mu;
std::unordered_map<const void *, bdattn_plan *> g_kept;

// Copies the plan's tables into the head of `dst` on `stream`, unless `dst` holds
// them already (kept by this plan) and `force` is false.
int upload(bdattn_plan *pl, void *dst, hipStream_t stream, bool force = false) {
  bdattn::Plan &p = pl->p;
  {
    std::lock_guard<std::mutex> kl(g_kept_mu);
    auto it = g_kept.find(dst);
    if (it != g_kept.end() && it->second == pl && !force) return BDATTN_OK;
    const uintptr_t lo = (uintptr_t)dst, hi = lo + p.image.size();
    for (auto k = g_kept.begin(); k != g_kept.end();) {
      const uintptr_t klo = (uintptr_t)k->first, khi = klo + k->second->p.image.size();
      if (k->second != pl && klo < hi && lo < khi) {   // those tables are about to be overwritten
        k->second->tables_at = nullptr;
        k = g_kept.erase(k);
      } else {
        ++k;
      }
    }
  }
  {
    std::lock_guard<std::mutex> lk(pl->mu);
    if (!p.pinned) {
      void *h = nullptr;
      HIP_CHECK(hipHostMalloc(&h, p.image.size(), hipHostMallocDefault), "hipHostMalloc");
      std::memcpy(h, p.image.data(), p.image.size());
      p.pinned = h;
    }
    p.used = true;
  }
  HIP_CHECK(hipMemcpyAsync(dst, p.pinned, p.image.size(), hipMemcpyHostToDevice, stream), "hipMemcpyAsync");
  return BDATTN_OK;
}

// Ends the plan's claim on its kept workspace, if any.
void release_kept(bdattn_plan *pl) {
  std::lock_guard<std::mutex> kl(g_kept_mu);
  if (pl->tables_at) {
    auto it = g_kept.find(pl->tables_at);
    if (it != g_kept.end() && it->second == pl) g_kept.erase(it);
    pl->tables_at = nullptr;
  }
}

const int32_t *img(const void *base, int64_t off) {
  return reinterpret_cast<const int32_t *>((const char *)base + off);
}

}  // namespace

namespace bdattn {
namespace abi {

int check_fwd_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k1,
                     const void *v1, const void *o, int32_t o_dtype, const float *lse) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  const bdattn::Plan &p = pl->p;
  CHECK(o_dtype == BDATTN_BF16 || o_dtype == BDATTN_F32, BDATTN_EUNSUPPORTED, "o_dtype must be BF16 or F32");
  const bool rows = p.n_q > 0;
  CHECK_PTR(q, rows);
  CHECK_PTR(o, rows);
  CHECK_PTR(lse, rows);
  int rc = check_shards(p, kv, false);
  if (rc != BDATTN_OK) return rc;
  CHECK_PTR(k1, p.n_seg[1] > 0);
  CHECK_PTR(v1, p.n_seg[1] > 0);
  return BDATTN_OK;
}

int check_fwd_args(const bdattn_plan *pl, const void *q, const void *k0, const void *v0, const void *k1,
                   const void *v1, const void *o, int32_t o_dtype, const float *lse) {
  const bdattn_kv_shards kv = one_buffer(k0, v0);
  return check_fwd_shards(pl, q, &kv, k1, v1, o, o_dtype, lse);
}

int launch_fwd_shards(const bdattn_plan *pl, const void *tables, const void *q, const bdattn_kv_shards &kv,
                      const void *k1, const void *v1, void *o, int32_t o_dtype, float *lse, hipStream_t s) {
  const bdattn::Plan &p = pl->p;
  const void *ws = tables;
  bdattn::FwdArgs a{};
  fill_shards(kv, a.sh, nullptr);
  a.k[0] = kv.k[0];
  a.k[1] = k1;
  a.v[0] = kv.v[0];
  a.v[1] = v1;
  a.n_seg[0] = (int32_t)p.n_seg[0];
  a.n_seg[1] = (int32_t)p.n_seg[1];
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.rows = img(ws, p.hdr.off_rows);
  a.items = img(ws, p.hdr.off_fwd);
  a.n_items = p.hdr.n_fwd;
  a.n_q = (int32_t)p.n_q;
  a.h_q = p.h_q;
  a.h_kv = p.h_kv;
  a.group = p.h_q / p.h_kv;
  a.o_f32 = o_dtype == BDATTN_F32;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  HIP_CHECK(bdattn::launch_fwd(a, p.d, s), "forward kernel");
  return BDATTN_OK;
}

int launch_fwd_on_tables(const bdattn_plan *pl, const void *tables, const void *q, const void *k0, const void *v0,
                         const void *k1, const void *v1, void *o, int32_t o_dtype, float *lse, hipStream_t s) {
  return launch_fwd_shards(pl, tables, q, one_buffer(k0, v0), k1, v1, o, o_dtype, lse, s);
}

int64_t fwd_table_bytes(const bdattn_plan *pl) { return pl->p.hdr.off_bq; }

}  // namespace abi
}  // namespace bdattn

namespace {

int run_fwd(const bdattn_plan *cpl, const void *q, const bdattn_kv_shards *kv, const void *k1, const void *v1,
            void *o, int32_t o_dtype, float *lse, void *ws, int64_t ws_bytes, void *stream) {
  bdattn_plan *pl = const_cast<bdattn_plan *>(cpl);
  int rc = bdattn::abi::check_fwd_shards(pl, q, kv, k1, v1, o, o_dtype, lse);
  if (rc != BDATTN_OK) return rc;
  rc = check_ws(pl->p, ws, ws_bytes);
  if (rc != BDATTN_OK) return rc;
  if (pl->p.n_q == 0) return BDATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  rc = upload(pl, ws, s);
  if (rc != BDATTN_OK) return rc;
  return bdattn::abi::launch_fwd_shards(pl, ws, q, *kv, k1, v1, o, o_dtype, lse, s);
}

int run_fwd(const bdattn_plan *cpl, const void *q, const void *k0, const void *v0, const void *k1,
            const void *v1, void *o, int32_t o_dtype, float *lse, void *ws, int64_t ws_bytes, void *stream) {
  const bdattn_kv_shards kv = one_buffer(k0, v0);
  return run_fwd(cpl, q, &kv, k1, v1, o, o_dtype, lse, ws, ws_bytes, stream);
}

int run_bwd(const bdattn_plan *cpl, const void *q, const bdattn_kv_shards *kv, const void *k1, const void *v1,
            const void *dout, const float *lse, const float *delta, float *dq, void *dk1, void *dv1, void *ws,
            int64_t ws_bytes, void *stream, bool do_dkdv = true, bool do_dq = true) {
  bdattn_plan *pl = const_cast<bdattn_plan *>(cpl);
  const bdattn::Plan &p = pl->p;
  const bool rows = p.n_q > 0;
  const bool any_keys = p.n_seg[0] + p.n_seg[1] > 0;
  const bool work = rows && any_keys;
  CHECK_PTR(q, work);
  CHECK_PTR(dout, work);
  CHECK_PTR(lse, work);
  CHECK_PTR(delta, work);
  CHECK_PTR(dq, work && do_dq);
  int rc = check_shards(p, kv, do_dkdv);
  if (rc != BDATTN_OK) return rc;
  CHECK_PTR(k1, p.n_seg[1] > 0);
  CHECK_PTR(v1, p.n_seg[1] > 0);
  CHECK_PTR(dk1, p.n_seg[1] > 0 && do_dkdv);
  CHECK_PTR(dv1, p.n_seg[1] > 0 && do_dkdv);
  rc = check_ws(p, ws, ws_bytes);
  if (rc != BDATTN_OK) return rc;
  if (!any_keys) return BDATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  rc = upload(pl, ws, s);
  if (rc != BDATTN_OK) return rc;
  bdattn::BwdArgs a{};
  fill_shards(*kv, a.sh, &a.gsh);
  a.k[0] = kv->k[0];
  a.k[1] = k1;
  a.v[0] = kv->v[0];
  a.v[1] = v1;
  a.dk[0] = kv->dk[0];
  a.dk[1] = dk1;
  a.dv[0] = kv->dv[0];
  a.dv[1] = dv1;
  a.n_seg[0] = (int32_t)p.n_seg[0];
  a.n_seg[1] = (int32_t)p.n_seg[1];
  a.q = q;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.rows = img(ws, p.hdr.off_rows);
  a.items = img(ws, p.hdr.off_fwd);
  a.bq = img(ws, p.hdr.off_bq);
  a.ktiles = img(ws, p.hdr.off_kt);
  a.list = img(ws, p.hdr.off_list);
  a.lrec = img(ws, p.hdr.off_lrec);
  a.n_items = rows ? p.hdr.n_fwd : 0;
  a.n_kt = p.hdr.n_kt;
  a.n_bq = p.hdr.n_bq;
  a.n_q = (int32_t)p.n_q;
  a.h_q = p.h_q;
  a.h_kv = p.h_kv;
  a.group = p.h_q / p.h_kv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.split = p.dkdv_split;
  for (int seg = 0; seg < 2; ++seg)
    a.part[seg] = p.dkdv_split > 1 ? reinterpret_cast<float *>((char *)ws + p.off_part[seg]) : nullptr;
  HIP_CHECK(bdattn::launch_bwd(a, p.d, s, do_dkdv, do_dq), "backward kernels");
  return BDATTN_OK;
}

int run_bwd(const bdattn_plan *cpl, const void *q, const void *k0, const void *v0, const void *k1,
            const void *v1, const void *dout, const float *lse, const float *delta, float *dq, void *dk0,
            void *dv0, void *dk1, void *dv1, void *ws, int64_t ws_bytes, void *stream, bool do_dkdv = true,
            bool do_dq = true) {
  const bdattn_kv_shards kv = one_buffer(k0, v0, dk0, dv0);
  return run_bwd(cpl, q, &kv, k1, v1, dout, lse, delta, dq, dk1, dv1, ws, ws_bytes, stream, do_dkdv, do_dq);
}

}  // namespace

extern "C" {

const char *bdattn_last_error(void) { return g_err.c_str(); }

int bdattn_plan_create(const bdattn_problem *pr, bdattn_plan **out) {
  if (!pr || !out) return fail(BDATTN_EINVAL, "problem or out is NULL");
  try {
    bdattn_plan *pl = new bdattn_plan;
    std::string e = bdattn::build_bdlm(pl->p, pr->clean_len, pr->block_size, pr->q_clean_offset, pr->q_clean_len,
                                       pr->owned_blocks, pr->n_owned, pr->kv_clean_offset, pr->kv_clean_len,
                                       pr->with_local_corrupt != 0, pr->h_q, pr->h_kv, pr->head_dim,
                                       pr->softmax_scale);
    if (!e.empty()) {
      delete pl;
      return fail_build(e);
    }
    *out = pl;
    return BDATTN_OK;
  } catch (const std::bad_alloc &) {
    return fail(BDATTN_EINVAL, "out of host memory building the plan");
  } catch (const std::exception &x) {
    return fail(BDATTN_EINVAL, x.what());
  }
}

int bdattn_plan_create_tasks(const int32_t *q_cu, const int32_t *k_cu, int32_t n_tasks, int32_t causal, int32_t h_q,
                             int32_t h_kv, int32_t head_dim, float scale, bdattn_plan **out) {
  if (!out) return fail(BDATTN_EINVAL, "out is NULL");
  try {
    bdattn_plan *pl = new bdattn_plan;
    std::string e = bdattn::build_tasks(pl->p, q_cu, k_cu, n_tasks, causal != 0, h_q, h_kv, head_dim, scale);
    if (!e.empty()) {
      delete pl;
      return fail_build(e);
    }
    *out = pl;
    return BDATTN_OK;
  } catch (const std::bad_alloc &) {
    return fail(BDATTN_EINVAL, "out of host memory building the plan");
  } catch (const std::exception &x) {
    return fail(BDATTN_EINVAL, x.what());
  }
}

int64_t bdattn_cad_split(const int32_t *cu, int32_t n_docs, int64_t max_pairs, int32_t *q_cu, int32_t *k_cu,
                         int32_t *kv_src, int64_t cap) {
  if (!cu) return fail(BDATTN_EINVAL, "cu_seqlens is NULL");
  if (n_docs < 0) return fail(BDATTN_EINVAL, "n_docs must be >= 0");
  if (max_pairs < 1) return fail(BDATTN_EINVAL, "max_pairs_per_task must be >= 1");
  if (cap < 0) return fail(BDATTN_EINVAL, "cap must be >= 0");
  if (cap > 0 && (!q_cu || !k_cu || !kv_src)) return fail(BDATTN_EINVAL, "output arrays are NULL");
  if (cu[0] != 0) return fail(BDATTN_EINVAL, "cu_seqlens[0] must be 0");
  for (int32_t s = 0; s < n_docs; ++s)
    if (cu[s + 1] < cu[s]) return fail(BDATTN_EINVAL, "cu_seqlens must be non-decreasing");
  int64_t total_ctx = 0;
  const int64_t n = bdattn::cad_split(cu, n_docs, max_pairs, nullptr, nullptr, nullptr, 0, &total_ctx);
  if (total_ctx > INT32_MAX / 2) return fail(BDATTN_EINVAL, "the tasks' key contexts exceed 2^30 rows");
  if (cap > 0) bdattn::cad_split(cu, n_docs, max_pairs, q_cu, k_cu, kv_src, cap, nullptr);
  return n;
}

int bdattn_plan_create_varlen(const int32_t *cu, int32_t n_seqs, int32_t causal, int32_t h_q, int32_t h_kv,
                              int32_t head_dim, float scale, bdattn_plan **out) {
  if (!out) return fail(BDATTN_EINVAL, "out is NULL");
  try {
    bdattn_plan *pl = new bdattn_plan;
    std::string e = bdattn::build_varlen(pl->p, cu, n_seqs, causal != 0, h_q, h_kv, head_dim, scale);
    if (!e.empty()) {
      delete pl;
      return fail_build(e);
    }
    *out = pl;
    return BDATTN_OK;
  } catch (const std::bad_alloc &) {
    return fail(BDATTN_EINVAL, "out of host memory building the plan");
  } catch (const std::exception &x) {
    return fail(BDATTN_EINVAL, x.what());
  }
}

void bdattn_plan_destroy(bdattn_plan *pl) {
  if (!pl) return;
  release_kept(pl);
  if (pl->p.pinned) {
    if (pl->p.used) (void)hipDeviceSynchronize();   // uploads may still read the pinned copy
    (void)hipHostFree(pl->p.pinned);
  }
  delete pl;
}

int64_t bdattn_plan_workspace_bytes(const bdattn_plan *pl) { return pl ? pl->p.ws_bytes : BDATTN_EINVAL; }

int bdattn_plan_keep_tables(bdattn_plan *pl, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (!ws) {
    release_kept(pl);
    return BDATTN_OK;
  }
  int rc = check_ws(pl->p, ws, ws_bytes);
  if (rc != BDATTN_OK) return rc;
  release_kept(pl);   // one kept workspace per plan
  rc = upload(pl, ws, (hipStream_t)stream, true);
  if (rc != BDATTN_OK) return rc;
  std::lock_guard<std::mutex> kl(g_kept_mu);
  g_kept[ws] = pl;
  pl->tables_at = ws;
  return BDATTN_OK;
}
int64_t bdattn_plan_useful_pairs(const bdattn_plan *pl) { return pl ? pl->p.useful_pairs : BDATTN_EINVAL; }
int64_t bdattn_plan_n_q(const bdattn_plan *pl) { return pl ? pl->p.n_q : BDATTN_EINVAL; }
int bdattn_plan_set_dkdv_split(bdattn_plan *pl, int32_t split) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (split < 0 || split > BDATTN_MAX_SPLIT)
    return fail(BDATTN_EINVAL, "split must be 0 (automatic) or 1.." + std::to_string(BDATTN_MAX_SPLIT));
  std::lock_guard<std::mutex> lk(pl->mu);
  if (pl->p.used) return fail(BDATTN_EINVAL, "the plan has already been used");
  if (split > 0 && bdattn::max_grid_items(pl->p, split) > BDATTN_MAX_GRID_ITEMS)
    return fail(BDATTN_EINVAL, "split too large: the dK/dV grid would exceed 2^32 work-items");
  bdattn::set_dkdv_split(pl->p, split);
  return BDATTN_OK;
}

int32_t bdattn_plan_dkdv_split(const bdattn_plan *pl) { return pl ? pl->p.dkdv_split : BDATTN_EINVAL; }

int bdattn_plan_heads(const bdattn_plan *pl, int32_t *h_q, int32_t *h_kv, int32_t *head_dim) {
  if (!pl || !h_q || !h_kv || !head_dim) return fail(BDATTN_EINVAL, "plan or output pointer is NULL");
  *h_q = pl->p.h_q;
  *h_kv = pl->p.h_kv;
  *head_dim = pl->p.d;
  return BDATTN_OK;
}

int64_t bdattn_plan_n_kv(const bdattn_plan *pl, int32_t seg) {
  if (!pl || seg < 0 || seg > 1) return fail(BDATTN_EINVAL, "bad plan or segment");
  return pl->p.n_seg[seg];
}

int64_t bdattn_plan_export(const bdattn_plan *pl, int32_t which, int32_t *out, int64_t cap) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  const bdattn::Plan &p = pl->p;
  const int32_t *src = nullptr;
  int64_t n = 0, w = 0;
  switch (which) {
    case 0: src = p.rows.data(); n = p.n_q; w = 4; break;
    case 1: src = reinterpret_cast<const int32_t *>(p.fwd.data()); n = (int64_t)p.fwd.size(); w = 12; break;
    case 2: src = reinterpret_cast<const int32_t *>(p.bq.data()); n = (int64_t)p.bq.size(); w = 12; break;
    case 3: src = reinterpret_cast<const int32_t *>(p.kt.data()); n = (int64_t)p.kt.size(); w = 4; break;
    case 4: src = p.list.data(); n = (int64_t)p.list.size(); w = 1; break;
    default: return fail(BDATTN_EINVAL, "which must be 0..4");
  }
  if (out && n > 0) std::memcpy(out, src, (size_t)(std::min(n, cap) * w * 4));
  return n;
}

int bdattn_fwd(const bdattn_plan *pl, const void *q, const void *k_clean, const void *v_clean, const void *k_corr,
               const void *v_corr, void *o, int32_t o_dtype, float *lse, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (pl->p.kind != 0) return fail(BDATTN_EINVAL, "plan is a varlen plan; use bdattn_varlen_fwd");
  return run_fwd(pl, q, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse, ws, ws_bytes, stream);
}

int bdattn_varlen_fwd(const bdattn_plan *pl, const void *q, const void *k, const void *v, void *o, int32_t o_dtype,
                      float *lse, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (pl->p.kind != 1) return fail(BDATTN_EINVAL, "plan is not a varlen plan; use bdattn_fwd");
  return run_fwd(pl, q, k, v, nullptr, nullptr, o, o_dtype, lse, ws, ws_bytes, stream);
}

int bdattn_bwd(const bdattn_plan *pl, const void *q, const void *k_clean, const void *v_clean, const void *k_corr,
               const void *v_corr, const void *dout, const float *lse, const float *delta, float *dq,
               void *dk_clean, void *dv_clean, void *dk_corr, void *dv_corr, void *ws, int64_t ws_bytes,
               void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (pl->p.kind != 0) return fail(BDATTN_EINVAL, "plan is a varlen plan; use bdattn_varlen_bwd");
  return run_bwd(pl, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq, dk_clean, dv_clean, dk_corr,
                 dv_corr, ws, ws_bytes, stream);
}

int bdattn_bwd_dkdv(const bdattn_plan *pl, const void *q, const void *k_clean, const void *v_clean,
                    const void *k_corr, const void *v_corr, const void *dout, const float *lse, const float *delta,
                    void *dk_clean, void *dv_clean, void *dk_corr, void *dv_corr, void *ws, int64_t ws_bytes,
                    void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_bwd(pl, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, nullptr, dk_clean, dv_clean, dk_corr,
                 dv_corr, ws, ws_bytes, stream, true, false);
}

int bdattn_bwd_dq(const bdattn_plan *pl, const void *q, const void *k_clean, const void *v_clean,
                  const void *k_corr, const void *v_corr, const void *dout, const float *lse, const float *delta,
                  float *dq_accum, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_bwd(pl, q, k_clean, v_clean, k_corr, v_corr, dout, lse, delta, dq_accum, nullptr, nullptr, nullptr,
                 nullptr, ws, ws_bytes, stream, false, true);
}

int bdattn_varlen_bwd(const bdattn_plan *pl, const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, const float *delta, float *dq, void *dk, void *dv, void *ws,
                      int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (pl->p.kind != 1) return fail(BDATTN_EINVAL, "plan is not a varlen plan; use bdattn_bwd");
  return run_bwd(pl, q, k, v, nullptr, nullptr, dout, lse, delta, dq, dk, dv, nullptr, nullptr, ws, ws_bytes,
                 stream);
}

int bdattn_fwd_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                      const void *v_corr, void *o, int32_t o_dtype, float *lse, void *ws, int64_t ws_bytes,
                      void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_fwd(pl, q, kv, k_corr, v_corr, o, o_dtype, lse, ws, ws_bytes, stream);
}

int bdattn_bwd_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                      const void *v_corr, const void *dout, const float *lse, const float *delta, float *dq_accum,
                      void *dk_corr, void *dv_corr, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_bwd(pl, q, kv, k_corr, v_corr, dout, lse, delta, dq_accum, dk_corr, dv_corr, ws, ws_bytes, stream);
}

int bdattn_bwd_dkdv_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                           const void *v_corr, const void *dout, const float *lse, const float *delta,
                           void *dk_corr, void *dv_corr, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_bwd(pl, q, kv, k_corr, v_corr, dout, lse, delta, nullptr, dk_corr, dv_corr, ws, ws_bytes, stream,
                 true, false);
}

int bdattn_bwd_dq_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k_corr,
                         const void *v_corr, const void *dout, const float *lse, const float *delta,
                         float *dq_accum, void *ws, int64_t ws_bytes, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  return run_bwd(pl, q, kv, k_corr, v_corr, dout, lse, delta, dq_accum, nullptr, nullptr, ws, ws_bytes, stream,
                 false, true);
}

int bdattn_bwd_prepare(const bdattn_plan *pl, const void *o, int32_t o_dtype, const void *dout, float *delta,
                       float *dq_accum, void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  const bdattn::Plan &p = pl->p;
  CHECK(o_dtype == BDATTN_BF16 || o_dtype == BDATTN_F32, BDATTN_EUNSUPPORTED, "o_dtype must be BF16 or F32");
  const bool rows = p.n_q > 0;
  CHECK_PTR(o, rows);
  CHECK_PTR(dout, rows);
  CHECK_PTR(delta, rows);
  if (dq_accum) CHECK_PTR(dq_accum, rows);
  if (!rows) return BDATTN_OK;
  bdattn::PrepArgs a{};
  a.o = o;
  a.dout = dout;
  a.o_f32 = o_dtype == BDATTN_F32;
  a.delta = delta;
  a.dq_zero = dq_accum;
  a.n_q = (int32_t)p.n_q;
  a.h_q = p.h_q;
  HIP_CHECK(bdattn::launch_prepare(a, p.d, (hipStream_t)stream), "prepare kernel");
  return BDATTN_OK;
}

int bdattn_cast_f32_bf16(const float *src, void *dst, int64_t n, void *stream) {
  CHECK(n >= 0, BDATTN_EINVAL, "n_elems must be >= 0");
  CHECK_PTR(src, n > 0);
  CHECK_PTR(dst, n > 0);
  if (n == 0) return BDATTN_OK;
  HIP_CHECK(bdattn::launch_cast_bf16(src, dst, n, (hipStream_t)stream), "cast kernel");
  return BDATTN_OK;
}

int bdattn_dq_finalize(const float *acc, void *dq, int64_t n, void *stream) {
  return bdattn_cast_f32_bf16(acc, dq, n, stream);
}

int bdattn_lse_merge(int32_t n_parts, const void *o_parts, int32_t part_dtype, const float *lse_parts,
                     int64_t n_rows, int32_t h, int32_t d, void *o_out, int32_t out_dtype, float *lse_out,
                     void *stream) {
  CHECK(n_parts >= 1, BDATTN_EINVAL, "n_parts must be >= 1");
  CHECK(n_rows >= 0 && h >= 1, BDATTN_EINVAL, "n_rows must be >= 0 and h >= 1");
  CHECK(d == 64 || d == 128, BDATTN_EUNSUPPORTED, "d must be 64 or 128");
  CHECK(part_dtype == BDATTN_BF16 || part_dtype == BDATTN_F32, BDATTN_EUNSUPPORTED, "part_dtype must be BF16 or F32");
  CHECK(out_dtype == BDATTN_BF16 || out_dtype == BDATTN_F32, BDATTN_EUNSUPPORTED, "out_dtype must be BF16 or F32");
  CHECK(n_rows * h * (d / 4) <= BDATTN_MAX_GRID_ITEMS, BDATTN_EUNSUPPORTED,
        "n_rows * h too large for one merge launch (grid beyond 2^32 work-items)");
  const bool any = n_rows > 0;
  CHECK_PTR(o_parts, any);
  CHECK_PTR(lse_parts, any);
  CHECK_PTR(o_out, any);
  CHECK_PTR(lse_out, any);
  if (!any) return BDATTN_OK;
  HIP_CHECK(bdattn::launch_merge(n_parts, o_parts, part_dtype == BDATTN_F32, lse_parts, n_rows, h, d, o_out,
                                 out_dtype == BDATTN_F32, lse_out, (hipStream_t)stream),
            "merge kernel");
  return BDATTN_OK;
}

}  // extern "C"
