// Host-side block-sparse tile scheduler.
//
// The BDLM mask gives every query row a contiguous legal key range in each key
// segment (a clean K/V range, and the local corrupted K/V), see the mask rules
// in bdattn.h ("rit.work explainer of CSBP", section on why conventional
// context parallelism sends extra data; "Block Parallelism For Efficient
// Distributed Long-Context Diffusion Language Model Training", English
// abstract).  The scheduler stores those ranges per row, tiles the rows, and
// keeps only the (query-tile, key-tile) pairs that hold a legal pair.  Each
// kept pair is marked full (no masked pair inside) or partial.  Tiles are
// ordered longest first so that the dispatcher's in-order launch approximates
// longest-processing-time balancing; with the early+late block pairing of the
// same explainer this keeps the per-tile cost spread small.
#include "plan.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <numeric>

namespace bdattn {

namespace {

std::atomic<uint64_t> g_next_id{1};

struct Region { int64_t begin, end; };   // query rows tiled together

void summarize(const std::vector<int32_t> &rows, int64_t q0, int64_t n, TileDesc &t) {
  t.q0 = (int32_t)q0;
  t.rows = (int32_t)n;
  for (int s = 0; s < 2; ++s) {
    int32_t lo_min = INT32_MAX, hi_max = INT32_MIN, lo_max = INT32_MIN, hi_min = INT32_MAX;
    bool any = false;
    for (int64_t r = q0; r < q0 + n; ++r) {
      int32_t lo = rows[r * 4 + 2 * s], hi = rows[r * 4 + 2 * s + 1];
      if (hi > lo) {
        any = true;
        lo_min = std::min(lo_min, lo);
        hi_max = std::max(hi_max, hi);
        lo_max = std::max(lo_max, lo);
        hi_min = std::min(hi_min, hi);
      } else {
        hi_min = 0;                 // an empty row: no key tile is full
        lo_max = std::max(lo_max, 0);
      }
    }
    if (!any) t.seg[s] = SegSummary{0, 0, 0, 0};
    else t.seg[s] = SegSummary{lo_min, lo_max, hi_min, hi_max};
  }
}

int32_t tiles_in(const SegSummary &s, int bn) {
  if (s.hi_max <= s.lo_min) return 0;
  int64_t a = s.lo_min / bn, b = (s.hi_max + bn - 1) / bn;
  return (int32_t)(b - a);
}

void tile_regions(Plan &p, const std::vector<Region> &regions) {
  p.fwd.clear();
  p.bq.clear();
  for (const Region &g : regions) {
    for (int64_t q0 = g.begin; q0 < g.end; q0 += BDATTN_FWD_BM) {
      TileDesc t{};
      summarize(p.rows, q0, std::min<int64_t>(BDATTN_FWD_BM, g.end - q0), t);
      // cost = key steps of the forward's walk
      t.cost = tiles_in(t.seg[0], BDATTN_FWD_STEP) + tiles_in(t.seg[1], BDATTN_FWD_STEP);
      p.fwd.push_back(t);
    }
    for (int64_t q0 = g.begin; q0 < g.end; q0 += BDATTN_BWD_BM) {
      TileDesc t{};
      summarize(p.rows, q0, std::min<int64_t>(BDATTN_BWD_BM, g.end - q0), t);
      t.cost = 0;
      p.bq.push_back(t);
    }
  }
  std::stable_sort(p.fwd.begin(), p.fwd.end(),
                   [](const TileDesc &a, const TileDesc &b) { return a.cost > b.cost; });
}

void build_bwd_lists(Plan &p) {
  const int bn = BDATTN_BWD_BN;
  int64_t nkt[2] = {(p.n_seg[0] + bn - 1) / bn, (p.n_seg[1] + bn - 1) / bn};
  int64_t n_tiles = nkt[0] + nkt[1];
  std::vector<int64_t> count(n_tiles + 1, 0);
  auto tile_index = [&](int s, int64_t k) { return (s == 0 ? 0 : nkt[0]) + k; };
  for (const TileDesc &t : p.bq)
    for (int s = 0; s < 2; ++s) {
      const SegSummary &g = t.seg[s];
      if (g.hi_max <= g.lo_min) continue;
      for (int64_t k = g.lo_min / bn; k * bn < g.hi_max; ++k) count[tile_index(s, k) + 1]++;
    }
  for (int64_t i = 0; i < n_tiles; ++i) count[i + 1] += count[i];
  p.list.assign(count[n_tiles], 0);
  std::vector<int64_t> fill(count.begin(), count.end() - 1);
  for (size_t qi = 0; qi < p.bq.size(); ++qi) {
    const TileDesc &t = p.bq[qi];
    for (int s = 0; s < 2; ++s) {
      const SegSummary &g = t.seg[s];
      if (g.hi_max <= g.lo_min) continue;
      for (int64_t k = g.lo_min / bn; k * bn < g.hi_max; ++k) {
        int64_t k0 = k * bn, k1 = k0 + bn;
        bool full = g.lo_max <= k0 && k1 <= g.hi_min;
        p.list[fill[tile_index(s, k)]++] = (int32_t)qi | (full ? INT32_MIN : 0);
      }
    }
  }
  p.lrec.assign(p.list.size() * 4, 0);
  for (size_t i = 0; i < p.list.size(); ++i) {
    const int32_t qi = p.list[i] & INT32_MAX;
    p.lrec[4 * i + 0] = p.bq[qi].q0;
    p.lrec[4 * i + 1] = p.bq[qi].rows;
    p.lrec[4 * i + 2] = p.list[i] < 0 ? 1 : 0;
    p.lrec[4 * i + 3] = qi;
  }
  p.kt.clear();
  for (int s = 0; s < 2; ++s)
    for (int64_t k = 0; k < nkt[s]; ++k) {
      int64_t i = tile_index(s, k);
      p.kt.push_back(KTile{s, (int32_t)(k * bn), (int32_t)count[i], (int32_t)count[i + 1]});
    }
  std::stable_sort(p.kt.begin(), p.kt.end(), [](const KTile &a, const KTile &b) {
    return (a.end - a.begin) > (b.end - b.begin);
  });
}

std::string finish(Plan &p) {
  p.useful_pairs = 0;
  for (int64_t r = 0; r < p.n_q; ++r)
    for (int s = 0; s < 2; ++s)
      p.useful_pairs += std::max<int64_t>(0, (int64_t)p.rows[r * 4 + 2 * s + 1] - p.rows[r * 4 + 2 * s]);
  build_bwd_lists(p);

  // Device image: header | rows | fwd items | bwd q-tiles | bwd k-tiles | bwd list | list records.
  ImageHeader &h = p.hdr;
  std::memset(&h, 0, sizeof(h));
  h.magic = BDATTN_IMAGE_MAGIC;
  h.n_q = (int32_t)p.n_q;
  h.n_fwd = (int32_t)p.fwd.size();
  h.n_bq = (int32_t)p.bq.size();
  h.n_kt = (int32_t)p.kt.size();
  h.n_list = (int32_t)p.list.size();
  h.n_seg0 = (int32_t)p.n_seg[0];
  h.n_seg1 = (int32_t)p.n_seg[1];
  int64_t off = align_up(sizeof(ImageHeader), BDATTN_ALIGN);
  h.off_rows = off;  off = align_up(off + (int64_t)p.rows.size() * 4, BDATTN_ALIGN);
  h.off_fwd = off;   off = align_up(off + (int64_t)p.fwd.size() * sizeof(TileDesc), BDATTN_ALIGN);
  h.off_bq = off;    off = align_up(off + (int64_t)p.bq.size() * sizeof(TileDesc), BDATTN_ALIGN);
  h.off_kt = off;    off = align_up(off + (int64_t)p.kt.size() * sizeof(KTile), BDATTN_ALIGN);
  h.off_list = off;  off = align_up(off + (int64_t)p.list.size() * 4, BDATTN_ALIGN);
  h.off_lrec = off;  off = align_up(off + (int64_t)p.lrec.size() * 4, BDATTN_ALIGN);
  h.image_bytes = off;
  p.image.assign(off, 0);
  std::memcpy(p.image.data(), &h, sizeof(h));
  if (!p.rows.empty()) std::memcpy(p.image.data() + h.off_rows, p.rows.data(), p.rows.size() * 4);
  if (!p.fwd.empty()) std::memcpy(p.image.data() + h.off_fwd, p.fwd.data(), p.fwd.size() * sizeof(TileDesc));
  if (!p.bq.empty()) std::memcpy(p.image.data() + h.off_bq, p.bq.data(), p.bq.size() * sizeof(TileDesc));
  if (!p.kt.empty()) std::memcpy(p.image.data() + h.off_kt, p.kt.data(), p.kt.size() * sizeof(KTile));
  if (!p.list.empty()) std::memcpy(p.image.data() + h.off_list, p.list.data(), p.list.size() * 4);
  if (!p.lrec.empty()) std::memcpy(p.image.data() + h.off_lrec, p.lrec.data(), p.lrec.size() * 4);

  set_dkdv_split(p, 0);
  if (max_grid_items(p, p.dkdv_split) > BDATTN_MAX_GRID_ITEMS)
    return "UNSUP:problem too large: a kernel's grid would exceed 2^32 work-items (split the rows or heads)";
  p.id = g_next_id.fetch_add(1);
  return "";
}

std::string check_heads(int32_t h_q, int32_t h_kv, int32_t d) {
  if (h_q <= 0 || h_kv <= 0) return "h_q and h_kv must be positive";
  if (h_q % h_kv) return "h_q must be a multiple of h_kv";
  if (d != 64 && d != 128) return "UNSUP:head_dim must be 64 or 128";
  return "";
}

}  // namespace

// Largest grid (work-items) of any kernel that runs on this plan, with `split`
// dK/dV workgroups per key tile: forward and dQ (one workgroup per query tile
// and q-head), dK/dV (per key tile, KV head and share), backward preparation
// (D/8 threads per row and q-head).
int64_t max_grid_items(const Plan &p, int32_t split) {
  const int64_t fwd = (int64_t)p.fwd.size() * p.h_q * 64 * BDATTN_FWD_WAVES;
  const int64_t dkdv = (int64_t)p.kt.size() * p.h_kv * split * BDATTN_DKDV_THREADS;
  const int64_t prep = p.n_q * p.h_q * (p.d / 8);
  return std::max(fwd, std::max(dkdv, prep));
}

// Splitting a key tile's walk over several workgroups only pays when the
// kernel would otherwise leave compute units idle: small problems have few key
// tiles, each with a long query-tile list, so one workgroup per key tile puts
// the whole list on one compute unit.
void set_dkdv_split(Plan &p, int32_t split) {
  const int64_t n_wg = (int64_t)p.kt.size() * p.h_kv;
  // bytes of one split's dK and dV partials over both key segments
  const int64_t part = 2 * (p.n_seg[0] + p.n_seg[1]) * p.h_kv * (int64_t)p.d * 4;
  if (split == 0) {
    int64_t longest = 0;
    for (const KTile &k : p.kt) longest = std::max<int64_t>(longest, (int64_t)(k.end - k.begin) * (p.h_q / p.h_kv));
    int64_t f = 1;
    if (n_wg > 0 && n_wg < BDATTN_SPLIT_TARGET / 2) {
      f = std::min<int64_t>(BDATTN_MAX_SPLIT, (BDATTN_SPLIT_TARGET + n_wg - 1) / n_wg);
      f = std::min<int64_t>(f, longest / BDATTN_SPLIT_MIN_ITERS);
      while (f > 1 && (f * part > BDATTN_SPLIT_MAX_BYTES || max_grid_items(p, (int32_t)f) > BDATTN_MAX_GRID_ITEMS))
        --f;
    }
    split = (int32_t)std::max<int64_t>(1, f);
  }
  p.dkdv_split = split;
  int64_t off = p.hdr.image_bytes;
  p.off_part[0] = p.off_part[1] = 0;
  if (split > 1) {
    for (int s = 0; s < 2; ++s) {
      p.off_part[s] = off;
      off = align_up(off + 2 * (int64_t)split * p.n_seg[s] * p.h_kv * p.d * 4, BDATTN_ALIGN);
    }
  }
  p.ws_bytes = off;
}

std::string build_bdlm(Plan &p, int64_t L, int32_t B, int64_t q_off, int64_t q_len,
                       const int64_t *owned, int64_t n_owned, int64_t kv_off, int64_t kv_len,
                       bool local, int32_t h_q, int32_t h_kv, int32_t d, float scale) {
  if (L <= 0 || B <= 0) return "clean_len and block_size must be positive";
  if (L % B) return "ALIGN:clean_len must be a multiple of block_size";
  if (q_off < 0 || q_len < 0 || q_off + q_len > L) return "clean query range outside [0, clean_len]";
  if (q_off % B || q_len % B) return "ALIGN:clean query range must be made of whole blocks";
  if (kv_off < 0 || kv_len < 0 || kv_off + kv_len > L) return "clean K/V range outside [0, clean_len]";
  if (kv_off % B || kv_len % B) return "ALIGN:clean K/V range must be made of whole blocks";
  if (n_owned < 0 || (n_owned > 0 && !owned)) return "owned_blocks is NULL";
  const int64_t nb = L / B;
  for (int64_t m = 0; m < n_owned; ++m)
    if (owned[m] < 0 || owned[m] >= nb) return "owned block id outside [0, clean_len / block_size)";
  std::string e = check_heads(h_q, h_kv, d);
  if (!e.empty()) return e;
  const int64_t n_q = q_len + n_owned * (int64_t)B;
  const int64_t n_corr = local ? n_owned * (int64_t)B : 0;
  if (n_q > INT32_MAX / 2 || kv_len > INT32_MAX / 2 || n_corr > INT32_MAX / 2)
    return "problem too large (row or key count beyond 2^30)";

  p.kind = 0;
  p.h_q = h_q; p.h_kv = h_kv; p.d = d;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  p.n_q = n_q;
  p.n_seg[0] = kv_len;
  p.n_seg[1] = n_corr;
  p.rows.assign(n_q * 4, 0);
  auto clamp_kv = [&](int64_t hi_global) {
    return (int32_t)std::min<int64_t>(kv_len, std::max<int64_t>(0, hi_global - kv_off));
  };
  for (int64_t i = 0; i < q_len; ++i) {                  // clean rows: block-causal
    int64_t pos = q_off + i;
    int32_t hi = clamp_kv((pos / B + 1) * B);
    p.rows[i * 4 + 1] = hi;
  }
  for (int64_t m = 0; m < n_owned; ++m) {                // corrupted rows: clean prefix + own block
    int32_t hi = clamp_kv(owned[m] * B);
    for (int64_t j = 0; j < B; ++j) {
      int64_t r = q_len + m * B + j;
      p.rows[r * 4 + 1] = hi;
      if (local) {
        p.rows[r * 4 + 2] = (int32_t)(m * B);
        p.rows[r * 4 + 3] = (int32_t)((m + 1) * B);
      }
    }
  }
  tile_regions(p, {Region{0, q_len}, Region{q_len, n_q}});
  return finish(p);
}

std::string build_tasks(Plan &p, const int32_t *q_cu, const int32_t *k_cu, int32_t n, bool causal, int32_t h_q,
                        int32_t h_kv, int32_t d, float scale) {
  if (!q_cu || !k_cu) return "q_cu / k_cu is NULL";
  if (n < 0) return "n_tasks must be >= 0";
  if (q_cu[0] != 0 || k_cu[0] != 0) return "q_cu[0] and k_cu[0] must be 0";
  for (int32_t t = 0; t < n; ++t)
    if (q_cu[t + 1] < q_cu[t] || k_cu[t + 1] < k_cu[t]) return "q_cu and k_cu must be non-decreasing";
  std::string e = check_heads(h_q, h_kv, d);
  if (!e.empty()) return e;
  const int64_t Tq = q_cu[n], Tk = k_cu[n];
  if (Tq > INT32_MAX / 2 || Tk > INT32_MAX / 2) return "problem too large";
  p.kind = 1;
  p.h_q = h_q; p.h_kv = h_kv; p.d = d;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  p.n_q = Tq;
  p.n_seg[0] = Tk;
  p.n_seg[1] = 0;
  p.rows.assign(Tq * 4, 0);
  std::vector<Region> regions;
  for (int32_t t = 0; t < n; ++t) {
    const int64_t q_len = q_cu[t + 1] - q_cu[t], k_len = k_cu[t + 1] - k_cu[t];
    for (int64_t i = 0; i < q_len; ++i) {
      // bottom-right alignment: the queries are the last q_len positions of the context
      const int64_t seen = causal ? std::min(k_len, std::max<int64_t>(0, k_len - q_len + i + 1)) : k_len;
      const int64_t r = q_cu[t] + i;
      p.rows[r * 4 + 0] = k_cu[t];
      p.rows[r * 4 + 1] = (int32_t)(k_cu[t] + seen);
    }
    if (q_len > 0) regions.push_back(Region{q_cu[t], q_cu[t + 1]});
  }
  tile_regions(p, regions);
  return finish(p);
}

int64_t cad_split(const int32_t *cu, int32_t n_docs, int64_t max_pairs, int32_t *q_cu, int32_t *k_cu,
                  int32_t *kv_src, int64_t cap, int64_t *total_ctx) {
  int64_t t = 0;
  if (cap > 0) {
    q_cu[0] = 0;
    k_cu[0] = 0;
  }
  int64_t qa = 0, ka = 0;
  for (int32_t s = 0; s < n_docs; ++s) {
    const int64_t start = cu[s], L = cu[s + 1] - cu[s];
    for (int64_t b = 0; b < L;) {
      // rows b .. e-1 of the document; row x sees the x + 1 keys of its prefix
      int64_t e = b + 1, pairs = b + 1;
      while (e < L && pairs + (e + 1) <= max_pairs) pairs += ++e;
      qa += e - b;
      ka += e;
      if (t < cap) {
        q_cu[t + 1] = (int32_t)qa;
        k_cu[t + 1] = (int32_t)ka;
        kv_src[t] = (int32_t)start;
      }
      ++t;
      b = e;
    }
  }
  if (total_ctx) *total_ctx = ka;
  return t;
}

std::string build_varlen(Plan &p, const int32_t *cu, int32_t n_seqs, bool causal, int32_t h_q,
                         int32_t h_kv, int32_t d, float scale) {
  if (!cu) return "cu_seqlens is NULL";
  if (n_seqs < 0) return "n_seqs must be >= 0";
  if (cu[0] != 0) return "cu_seqlens[0] must be 0";
  for (int32_t i = 0; i < n_seqs; ++i)
    if (cu[i + 1] < cu[i]) return "cu_seqlens must be non-decreasing";
  std::string e = check_heads(h_q, h_kv, d);
  if (!e.empty()) return e;
  const int64_t T = cu[n_seqs];
  if (T > INT32_MAX / 2) return "problem too large";
  p.kind = 1;
  p.h_q = h_q; p.h_kv = h_kv; p.d = d;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  p.n_q = T;
  p.n_seg[0] = T;
  p.n_seg[1] = 0;
  p.rows.assign(T * 4, 0);
  std::vector<Region> regions;
  for (int32_t s = 0; s < n_seqs; ++s) {
    for (int64_t r = cu[s]; r < cu[s + 1]; ++r) {
      p.rows[r * 4 + 0] = cu[s];
      p.rows[r * 4 + 1] = causal ? (int32_t)(r + 1) : cu[s + 1];
    }
    if (cu[s + 1] > cu[s]) regions.push_back(Region{cu[s], cu[s + 1]});
  }
  tile_regions(p, regions);
  return finish(p);
}

}  // namespace bdattn
