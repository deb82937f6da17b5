// Host-only driver for the AddressSanitizer / UndefinedBehaviorSanitizer build
// of the tile scheduler (plan.cpp) and the C ABI's validation (capi.cpp).
//
// It builds many random BDLM, varlen and task plans, checks each plan's
// per-row key ranges against a brute-force evaluation of the mask rules and the
// exported tables against each other, runs the document splitter, and drives
// every rejection path of the compute entry points with fake device addresses.
// Every compute call made here must fail validation before any HIP call: the
// kernel launchers are stubs that abort, and a status of BDATTN_EHIP means a
// HIP call was reached.  Exit status 0 and a final "ok" line mean every check
// passed (the sanitizers abort on their own findings).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "bdattn.h"

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t rnd() {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}
int64_t rnd_in(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

int g_fail = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      std::fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                    \
      std::fprintf(stderr, " [%s]\n", bdattn_last_error()); \
      if (++g_fail > 20) std::exit(1);                      \
    }                                                       \
  } while (0)

std::vector<int32_t> export_table(const bdattn_plan *p, int which, int width) {
  const int64_t n = bdattn_plan_export(p, which, nullptr, 0);
  std::vector<int32_t> out((size_t)(n * width) + 1, -7);
  bdattn_plan_export(p, which, out.data(), n);
  out.resize((size_t)(n * width));
  return out;
}

// Row bounds against a brute-force key predicate; tables against each other.
template <class Legal>
void check_plan(const bdattn_plan *p, int64_t n_q, int64_t n0, int64_t n1, Legal legal) {
  EXPECT(bdattn_plan_n_q(p) == n_q, "n_q");
  EXPECT(bdattn_plan_n_kv(p, 0) == n0 && bdattn_plan_n_kv(p, 1) == n1, "n_kv");
  const std::vector<int32_t> rows = export_table(p, 0, 4);
  int64_t pairs = 0;
  for (int64_t r = 0; r < n_q; ++r)
    for (int s = 0; s < 2; ++s) {
      const int32_t lo = rows[r * 4 + 2 * s], hi = rows[r * 4 + 2 * s + 1];
      const int64_t nk = s ? n1 : n0;
      for (int64_t k = 0; k < nk; ++k) {
        const bool want = legal(r, s, k);
        const bool got = lo <= k && k < hi;
        if (want != got) {
          EXPECT(false, "row %lld segment %d key %lld: mask %d, plan range [%d, %d)", (long long)r, s,
                 (long long)k, (int)want, lo, hi);
          return;
        }
        pairs += want;
      }
    }
  EXPECT(bdattn_plan_useful_pairs(p) == pairs, "useful pairs %lld vs %lld", (long long)bdattn_plan_useful_pairs(p),
         (long long)pairs);
  // forward tiles: every row exactly once
  const std::vector<int32_t> fwd = export_table(p, 1, 12);
  std::vector<int> seen((size_t)n_q, 0);
  for (size_t i = 0; i < fwd.size(); i += 12) {
    EXPECT(fwd[i] >= 0 && fwd[i + 1] > 0 && fwd[i] + fwd[i + 1] <= n_q, "fwd tile bounds");
    for (int32_t r = fwd[i]; r < fwd[i] + fwd[i + 1] && r < n_q; ++r) seen[(size_t)r]++;
  }
  for (int64_t r = 0; r < n_q; ++r) EXPECT(seen[(size_t)r] == 1, "row %lld in %d forward tiles", (long long)r, seen[r]);
  // backward lists: entries name existing query tiles; a key tile's rows all lie in its list
  const std::vector<int32_t> bq = export_table(p, 2, 12), kt = export_table(p, 3, 4), list = export_table(p, 4, 1);
  const int64_t n_bq = (int64_t)bq.size() / 12;
  for (size_t i = 0; i < kt.size(); i += 4) {
    const int32_t seg = kt[i], k0 = kt[i + 1], b = kt[i + 2], e = kt[i + 3];
    EXPECT(seg == 0 || seg == 1, "key tile segment");
    EXPECT(0 <= b && b <= e && e <= (int32_t)list.size(), "key tile list range");
    std::vector<char> in_list((size_t)n_bq, 0);
    for (int32_t j = b; j < e && j < (int32_t)list.size(); ++j) {
      const int32_t qi = list[(size_t)j] & INT32_MAX;
      EXPECT(qi >= 0 && qi < n_bq, "list entry names query tile %d of %lld", qi, (long long)n_bq);
      if (qi >= 0 && qi < n_bq) in_list[(size_t)qi] = 1;
    }
    const int64_t nk = seg ? n1 : n0;
    for (int64_t qi = 0; qi < n_bq; ++qi) {
      if (in_list[(size_t)qi]) continue;
      for (int32_t r = bq[qi * 12]; r < bq[qi * 12] + bq[qi * 12 + 1]; ++r)
        for (int64_t k = k0; k < k0 + 128 && k < nk; ++k)
          if (legal(r, seg, k)) {
            EXPECT(false, "row %d attends key %lld of tile %d but its query tile is not listed", r, (long long)k, k0);
            return;
          }
    }
  }
}

void fuzz_bdlm(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int32_t B = (int32_t)rnd_in(1, 48);
    const int64_t nb = rnd_in(1, 40), L = nb * B;
    const int64_t qb0 = rnd_in(0, nb), qb1 = rnd_in(qb0, nb);
    const int64_t kb0 = rnd_in(0, nb), kb1 = rnd_in(kb0, nb);
    std::vector<int64_t> owned;
    for (int64_t b = 0; b < nb; ++b)
      if (rnd() % 3 == 0) owned.push_back(b);
    for (size_t i = owned.size(); i > 1; --i) std::swap(owned[i - 1], owned[(size_t)rnd_in(0, (int64_t)i - 1)]);
    const int32_t h_kv = (int32_t)rnd_in(1, 3), G = (int32_t)rnd_in(1, 4);
    bdattn_problem pr{};
    pr.clean_len = L;
    pr.block_size = B;
    pr.q_clean_offset = qb0 * B;
    pr.q_clean_len = (qb1 - qb0) * B;
    pr.owned_blocks = owned.data();
    pr.n_owned = (int64_t)owned.size();
    pr.kv_clean_offset = kb0 * B;
    pr.kv_clean_len = (kb1 - kb0) * B;
    pr.with_local_corrupt = (int32_t)(rnd() % 2);
    pr.h_q = h_kv * G;
    pr.h_kv = h_kv;
    pr.head_dim = rnd() % 2 ? 64 : 128;
    bdattn_plan *p = nullptr;
    EXPECT(bdattn_plan_create(&pr, &p) == BDATTN_OK, "valid BDLM problem rejected");
    if (!p) continue;
    const int64_t q_len = pr.q_clean_len, n_corr = pr.n_owned * B;
    auto legal = [&](int64_t r, int s, int64_t k) -> bool {
      if (r < q_len) {                          // clean row: block-causal over clean keys
        if (s) return false;
        const int64_t pos = pr.q_clean_offset + r, t = pr.kv_clean_offset + k;
        return t / B <= pos / B;
      }
      const int64_t m = (r - q_len) / B;      // corrupted slot m of block owned[m]
      if (s == 0) return pr.kv_clean_offset + k < owned[(size_t)m] * B;
      return k / B == m;
    };
    check_plan(p, q_len + n_corr, pr.kv_clean_len, pr.with_local_corrupt ? n_corr : 0, legal);
    const int32_t split = (int32_t)rnd_in(-1, 9);
    const int rc = bdattn_plan_set_dkdv_split(p, split);
    EXPECT((split >= 0 && split <= 8) ? rc == BDATTN_OK : rc == BDATTN_EINVAL, "set_dkdv_split(%d) -> %d", split, rc);
    EXPECT(bdattn_plan_workspace_bytes(p) > 0 && bdattn_plan_workspace_bytes(p) % 256 == 0, "workspace size");
    bdattn_plan_destroy(p);
  }
}

void fuzz_varlen_and_tasks(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int n = (int)rnd_in(0, 6);
    std::vector<int32_t> cu(1, 0), kc(1, 0);
    for (int i = 0; i < n; ++i) {
      cu.push_back(cu.back() + (int32_t)rnd_in(0, 300));
      kc.push_back(kc.back() + (int32_t)rnd_in(0, 400));
    }
    const int causal = (int)(rnd() % 2);
    bdattn_plan *p = nullptr;
    EXPECT(bdattn_plan_create_varlen(cu.data(), n, causal, 4, 2, 128, 0.f, &p) == BDATTN_OK, "varlen rejected");
    if (p) {
      auto shard = [&](int64_t x) { int s = 0; while (cu[(size_t)s + 1] <= x) ++s; return s; };
      auto legal = [&](int64_t r, int s, int64_t k) -> bool {
        if (s) return false;
        const int sr = shard(r), sk = shard(k);
        return sr == sk && (!causal || k <= r);
      };
      check_plan(p, cu.back(), cu.back(), 0, legal);
      bdattn_plan_destroy(p);
    }
    p = nullptr;
    EXPECT(bdattn_plan_create_tasks(cu.data(), kc.data(), n, causal, 4, 2, 64, 0.f, &p) == BDATTN_OK,
           "tasks rejected");
    if (p) {
      auto task_of = [&](const std::vector<int32_t> &c, int64_t x) { int s = 0; while (c[(size_t)s + 1] <= x) ++s; return s; };
      auto legal = [&](int64_t r, int s, int64_t k) -> bool {
        if (s) return false;
        const int t = task_of(cu, r);
        if (k < kc[(size_t)t] || k >= kc[(size_t)t + 1]) return false;
        if (!causal) return true;
        const int64_t ql = cu[(size_t)t + 1] - cu[(size_t)t], kl = kc[(size_t)t + 1] - kc[(size_t)t];
        return k - kc[(size_t)t] <= kl - ql + (r - cu[(size_t)t]);   // bottom-right alignment
      };
      check_plan(p, cu.back(), kc.back(), 0, legal);
      bdattn_plan_destroy(p);
    }
    // document splitter: runs of rows, prefix contexts, bounded pairs
    const int64_t maxp = rnd_in(1, 20000);
    const int64_t nt = bdattn_cad_split(cu.data(), n, maxp, nullptr, nullptr, nullptr, 0);
    EXPECT(nt >= 0, "cad_split count");
    if (nt > 0) {
      std::vector<int32_t> q_cu((size_t)nt + 1), k_cu((size_t)nt + 1), src((size_t)nt);
      EXPECT(bdattn_cad_split(cu.data(), n, maxp, q_cu.data(), k_cu.data(), src.data(), nt) == nt, "cad_split");
      EXPECT(q_cu[(size_t)nt] == cu.back(), "tasks cover every row");
      for (int64_t t = 0; t < nt; ++t) {
        const int64_t ql = q_cu[(size_t)t + 1] - q_cu[(size_t)t], kl = k_cu[(size_t)t + 1] - k_cu[(size_t)t];
        EXPECT(ql >= 1 && kl >= ql, "task %lld shape", (long long)t);
        // the context ends at the task's last row: its document offset is q_cu - src + ql
        EXPECT(q_cu[(size_t)t] - src[(size_t)t] + ql == kl, "task %lld context is its prefix", (long long)t);
        const int64_t first = kl - ql;   // row index (in its document) of the task's first row
        const int64_t pairs = ql * (first + 1) + ql * (ql - 1) / 2;
        EXPECT(pairs <= maxp || ql == 1, "task %lld has %lld pairs > %lld", (long long)t, (long long)pairs,
               (long long)maxp);
      }
    }
  }
}

// Every compute entry point, with one bad argument at a time: each call must
// return its status before any HIP call (EHIP would mean one was reached).
void rejections() {
  std::vector<int64_t> owned = {3, 1};
  bdattn_problem pr{};
  pr.clean_len = 256; pr.block_size = 32; pr.q_clean_offset = 64; pr.q_clean_len = 64;
  pr.owned_blocks = owned.data(); pr.n_owned = 2; pr.kv_clean_offset = 0; pr.kv_clean_len = 128;
  pr.with_local_corrupt = 1; pr.h_q = 4; pr.h_kv = 2; pr.head_dim = 128;
  bdattn_plan *p = nullptr;
  EXPECT(bdattn_plan_create(&pr, &p) == BDATTN_OK, "reference problem");
  if (!p) return;
  void *g = reinterpret_cast<void *>(uintptr_t(1) << 20);   // never dereferenced
  void *mis = reinterpret_cast<void *>((uintptr_t(1) << 20) + 8);
  float *gf = static_cast<float *>(g), *mf = static_cast<float *>(mis);
  const int64_t ws = bdattn_plan_workspace_bytes(p);
  EXPECT(bdattn_fwd(p, nullptr, g, g, g, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EINVAL, "fwd q NULL");
  EXPECT(bdattn_fwd(p, mis, g, g, g, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EALIGN, "fwd q misaligned");
  EXPECT(bdattn_fwd(p, g, g, g, nullptr, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EINVAL, "fwd k_corr");
  EXPECT(bdattn_fwd(p, g, g, g, g, g, g, 9, gf, g, ws, nullptr) == BDATTN_EUNSUPPORTED, "fwd dtype");
  EXPECT(bdattn_fwd(p, g, g, g, g, g, g, BDATTN_F32, gf, g, ws - 1, nullptr) == BDATTN_EWORKSPACE, "fwd ws");
  EXPECT(bdattn_fwd(p, g, g, g, g, g, g, BDATTN_F32, gf, mis, ws, nullptr) == BDATTN_EALIGN, "fwd ws align");
  EXPECT(bdattn_fwd(nullptr, g, g, g, g, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EINVAL, "fwd plan");
  EXPECT(bdattn_varlen_fwd(p, g, g, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EINVAL, "varlen fwd on BDLM");
  EXPECT(bdattn_bwd(p, g, g, g, g, g, g, gf, gf, gf, g, g, g, nullptr, g, ws, nullptr) == BDATTN_EINVAL, "bwd dv_corr");
  EXPECT(bdattn_bwd(p, g, g, g, g, g, g, mf, gf, gf, g, g, g, g, g, ws, nullptr) == BDATTN_EALIGN, "bwd lse");
  EXPECT(bdattn_bwd(p, g, g, g, g, g, g, gf, gf, gf, g, g, g, g, g, 16, nullptr) == BDATTN_EWORKSPACE, "bwd ws");
  EXPECT(bdattn_bwd_dkdv(p, g, g, g, g, g, g, gf, gf, nullptr, g, g, g, g, ws, nullptr) == BDATTN_EINVAL, "dkdv");
  EXPECT(bdattn_bwd_dq(p, g, g, g, g, g, g, gf, gf, nullptr, g, ws, nullptr) == BDATTN_EINVAL, "dq accum");
  EXPECT(bdattn_bwd_prepare(p, g, 5, g, gf, gf, nullptr) == BDATTN_EUNSUPPORTED, "prepare dtype");
  EXPECT(bdattn_bwd_prepare(p, g, BDATTN_BF16, g, nullptr, gf, nullptr) == BDATTN_EINVAL, "prepare delta");
  EXPECT(bdattn_lse_merge(0, g, BDATTN_F32, gf, 10, 2, 128, g, BDATTN_BF16, gf, nullptr) == BDATTN_EINVAL, "merge n");
  EXPECT(bdattn_lse_merge(2, g, BDATTN_F32, gf, 10, 2, 96, g, BDATTN_BF16, gf, nullptr) == BDATTN_EUNSUPPORTED, "d");
  EXPECT(bdattn_lse_merge(2, g, BDATTN_F32, gf, int64_t(1) << 28, 2, 128, g, BDATTN_BF16, gf, nullptr) ==
             BDATTN_EUNSUPPORTED, "merge grid");
  EXPECT(bdattn_dq_finalize(nullptr, g, 10, nullptr) == BDATTN_EINVAL, "finalize");
  EXPECT(bdattn_cast_f32_bf16(gf, mis, 10, nullptr) == BDATTN_EALIGN, "cast");
  EXPECT(bdattn_plan_export(p, 7, nullptr, 0) == BDATTN_EINVAL, "export which");
  EXPECT(bdattn_plan_keep_tables(nullptr, g, ws, nullptr) == BDATTN_EINVAL, "keep plan NULL");
  EXPECT(bdattn_plan_keep_tables(p, mis, ws, nullptr) == BDATTN_EALIGN, "keep misaligned");
  EXPECT(bdattn_plan_keep_tables(p, g, ws - 1, nullptr) == BDATTN_EWORKSPACE, "keep small");
  EXPECT(bdattn_plan_keep_tables(p, nullptr, 0, nullptr) == BDATTN_OK, "keep release");
  int32_t a, b, c;
  EXPECT(bdattn_plan_heads(p, &a, &b, &c) == BDATTN_OK && a == 4 && b == 2 && c == 128, "heads");
  EXPECT(bdattn_plan_heads(p, nullptr, &b, &c) == BDATTN_EINVAL, "heads NULL");
  bdattn_plan_destroy(p);
  // problems beyond the size limits, and malformed ones
  bdattn_problem big = pr;
  big.clean_len = int64_t(1) << 31; big.block_size = 1 << 20; big.q_clean_offset = 0; big.q_clean_len = int64_t(1) << 30;
  big.n_owned = 0; big.owned_blocks = nullptr; big.kv_clean_len = 1 << 20;
  p = nullptr;
  EXPECT(bdattn_plan_create(&big, &p) == BDATTN_EINVAL && !p, "2^30 rows");
  bdattn_problem bad = pr;
  bad.owned_blocks = nullptr;
  EXPECT(bdattn_plan_create(&bad, &p) == BDATTN_EINVAL, "owned NULL");
  bad = pr; bad.q_clean_offset = 16;
  EXPECT(bdattn_plan_create(&bad, &p) == BDATTN_EALIGN, "misaligned q range");
  bad = pr; bad.head_dim = 96;
  EXPECT(bdattn_plan_create(&bad, &p) == BDATTN_EUNSUPPORTED, "head dim");
  EXPECT(bdattn_plan_create(nullptr, &p) == BDATTN_EINVAL, "problem NULL");
  const int32_t cu_bad[3] = {0, 5, 3};
  EXPECT(bdattn_plan_create_varlen(cu_bad, 2, 1, 4, 2, 128, 0.f, &p) == BDATTN_EINVAL, "varlen decreasing");
  const int32_t cu_big[2] = {0, 1 << 30};
  EXPECT(bdattn_plan_create_varlen(cu_big, 1, 1, 4, 2, 128, 0.f, &p) == BDATTN_EINVAL, "varlen 2^30");
  EXPECT(bdattn_cad_split(cu_bad, 2, 10, nullptr, nullptr, nullptr, 0) == BDATTN_EINVAL, "cad decreasing");
  bdattn_plan_destroy(nullptr);
}

// Random buffer tables of the *_shards entry points against a brute-force
// reading of their rules: a valid table must get as far as the workspace check
// (the workspace is one byte short), so no call reaches a launch.
void fuzz_shards(int iters) {
  std::vector<int64_t> owned = {20, 3};
  bdattn_problem pr{};
  pr.clean_len = 1024; pr.block_size = 32; pr.q_clean_offset = 128; pr.q_clean_len = 256;
  pr.owned_blocks = owned.data(); pr.n_owned = 2; pr.kv_clean_offset = 128; pr.kv_clean_len = 640;
  pr.with_local_corrupt = 1; pr.h_q = 4; pr.h_kv = 2; pr.head_dim = 64;
  bdattn_plan *p = nullptr;
  EXPECT(bdattn_plan_create(&pr, &p) == BDATTN_OK, "shard problem");
  if (!p) return;
  const int64_t n0 = bdattn_plan_n_kv(p, 0), ws = bdattn_plan_workspace_bytes(p);
  EXPECT(n0 == 640, "shard problem keys");
  void *g = reinterpret_cast<void *>(uintptr_t(1) << 20);
  float *gf = static_cast<float *>(g);
  const int64_t lens[] = {0, -128, 64, 100, 128, 192, 256, 320, 384, 640, 768, int64_t(1) << 40, 130};
  for (int it = 0; it < iters; ++it) {
    bdattn_kv_shards t{};
    t.n_shards = (int32_t)rnd_in(-2, 20);
    t.shard_len = lens[rnd_in(0, (int64_t)(sizeof(lens) / sizeof(lens[0])) - 1)];
    for (int i = 0; i < BDATTN_MAX_SHARDS; ++i) t.k[i] = t.v[i] = t.dk[i] = t.dv[i] = g;
    const bool grads = rnd_in(0, 1) == 1;
    // at most one bad entry: field f of entry e, NULL or misaligned
    const int f = (int)rnd_in(0, 4), e = (int)rnd_in(0, BDATTN_MAX_SHARDS - 1);
    const bool null_ptr = rnd_in(0, 1) == 1;
    void *bad = null_ptr ? nullptr : reinterpret_cast<void *>((uintptr_t(1) << 20) + 4);
    if (f == 0) t.k[e] = bad;
    if (f == 1) t.v[e] = bad;
    if (f == 2) t.dk[e] = bad;
    if (f == 3) t.dv[e] = bad;
    int want = BDATTN_EWORKSPACE;
    const int n = t.n_shards;
    if (n < 1 || n > BDATTN_MAX_SHARDS) {
      want = BDATTN_EINVAL;
    } else if (n > 1 && (t.shard_len <= 0 || t.shard_len % BDATTN_SHARD_ALIGN != 0)) {
      want = BDATTN_EALIGN;
    } else if (n > 1 && !(t.shard_len < n0 && (n - 1) * t.shard_len < n0 && n0 <= n * t.shard_len)) {
      want = BDATTN_EINVAL;
    } else if (f < 4 && e < n && (f < 2 || grads)) {
      want = null_ptr ? BDATTN_EINVAL : BDATTN_EALIGN;
    }
    const int rc = grads ? bdattn_bwd_dkdv_shards(p, g, &t, g, g, g, gf, gf, g, g, g, ws - 1, nullptr)
                         : bdattn_fwd_shards(p, g, &t, g, g, g, BDATTN_F32, gf, g, ws - 1, nullptr);
    EXPECT(rc == want, "shard table n=%d len=%lld field %d entry %d %s: got %d, want %d", n,
           (long long)t.shard_len, f, e, null_ptr ? "NULL" : "misaligned", rc, want);
  }
  EXPECT(bdattn_fwd_shards(p, g, nullptr, g, g, g, BDATTN_F32, gf, g, ws, nullptr) == BDATTN_EINVAL, "kv NULL");
  bdattn_plan_destroy(p);
}

}  // namespace

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 300;
  fuzz_bdlm(iters);
  fuzz_varlen_and_tasks(iters);
  rejections();
  fuzz_shards(iters * 10);
  if (g_fail) {
    std::printf("%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ok: %d random BDLM plans, %d varlen/task/splitter cases, %d shard tables, every rejection path\n",
              iters, iters, iters * 10);
  return 0;
}
