// Backward of BDLM-masked core attention on gfx950, for one K/V range.
//
// Gradients flow to the queries, the clean K/V range and the local corrupted
// K/V ("rit.work explainer of CSBP": conventional context parallelism returns
// the K/V gradients, CSBP returns only the clean ones and keeps the corrupted
// ones with their block).  With the MERGED log-sum-exp of every row the
// probabilities of a range are exact, so per-range backwards add up to the
// unsharded one ("Block Parallelism For Efficient Distributed Long-Context
// Diffusion Language Model Training", English abstract: training semantics
// are preserved).  With P = exp(S - LSE) and dS = P o (dO V^T - delta):
//
//   dkdv_kernel (key-major): one workgroup = 128 keys of one KV head.  It walks
//     the query tiles (64 rows) that attend its keys, for every q-head of the
//     group.  Eight waves, two per SIMD: four "dV waves" (32 keys each, K in
//     registers) compute S = Q K^T, P and dV^T += dO^T P; four "dK waves" on
//     the same keys (V in registers) compute dP = dO V^T, take P from the dV
//     waves through LDS, and form dS and dK^T += Q^T dS.  The dV waves run one
//     query tile ahead, so the two roles share no data inside an iteration and
//     one barrier per tile suffices.  Each wave keeps one accumulator and one
//     operand set, so two waves fit every SIMD; the MFMA work per pair is that
//     of a fused kernel.  S and dP put one key per lane, so P and dS feed the
//     accumulating MFMAs straight from the C registers (dO^T and Q^T come from
//     transpose reads).  dK and dV are summed over the group in registers and
//     written once.
//   dq_kernel (query-major, shaped like the forward): one workgroup = 32 rows
//     per wave of one q-head.  S^T = K Q^T and dP^T = V dO^T put one query per
//     lane (its LSE and delta are scalars), and dQ^T += K^T dS^T takes dS^T
//     from the C registers and K^T from transpose reads of the K tile.  dQ is
//     owned by one workgroup per call: it is added to the fp32 accumulator
//     without atomics.
// The split recomputes S and dP once more than a fused kernel, but removes the
// fp32 atomics a fused key-major kernel needs for dQ (about one per useful pair
// and head), which the L2 executes far slower than the MFMA work they replace.
#include <cfloat>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace bdattn {
namespace {

// Static LDS of the dK/dV kernel.  Query tiles (Q) pass through three buffers and
// dO tiles through two, because the dV waves run one tile ahead of the dK waves:
// in iteration i they read Q(i + 1) and dO(i), the dK waves read dO(i) and Q(i),
// and the loads of Q(i + 2) and dO(i + 1) are in flight.  P goes from the dV to
// the dK waves through two buffers for the same reason.
template <int D>
struct DkdvLds {
  char *q[3], *d[2];
  float (*sq[3])[BDATTN_BWD_BM];   // per Q tile: -LSE log2(e), lo, hi of its rows
  float *sd[2];                    // per dO tile: delta of its rows
  f32x4 *pb[2];                    // P of one tile: [wave][row half][key tile][register quad][lane]
};

// The loop of one dkdv role.  A wave owns KT column tiles of 32 keys, so every
// Q or dO operand it reads from LDS feeds KT MFMAs.  Per iteration i (one query
// tile of one head), with P(i) made by the dV waves in iteration i - 1 and left
// in LDS:
//   role 0 (dV waves, hold K): S = Q(i+1) K^T and P(i+1) = exp(S - LSE) on the
//            legal pairs, stored to LDS (fp32, C-register layout) and kept in
//            registers as bf16; dV^T += dO(i)^T P(i) from the registers.
//   role 1 (dK waves, hold V): dP = dO(i) V^T; P(i) from LDS (same lane <-> key
//            map); dS = P o (dP - delta), dK^T += Q(i)^T dS.
// The roles share no data inside an iteration, so one barrier per iteration
// suffices.
template <int D, int KT, int ROLE, bool SPLIT>
__device__ __forceinline__ void dkdv_role(const BwdArgs &a, int s, int k0, int lb, int t0, int nt, int chunk,
                                          int kvh, int wave, int lane, const DkdvLds<D> &L) {
  constexpr int BM = BDATTN_BWD_BM;
  constexpr int NWR = 4 / KT;   // waves per role
  constexpr int NC = D / 16, ND = D / 32;
  const int j = lane & 31, g = lane >> 5;
  const int kw = wave % NWR;
  int key[KT];
  bool kvalid[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    key[kt] = k0 + (kw * KT + kt) * 32 + j;
    kvalid[kt] = key[kt] < a.n_seg[s];
  }
  const int G = a.group;

  // The buffer of this key tile (a key tile never straddles two) and the first
  // key of that buffer.
  const void *kbuf, *vbuf;
  const int kbase = k0 - seg_buffer<SPLIT>(a, s, k0, kbuf, vbuf);
  // K (dV waves) or V (dK waves) as B operands (lane = key column, k = head dim).
  bf16x8 kvf[KT][NC];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int64_t off = ((int64_t)(kvalid[kt] ? key[kt] - kbase : 0) * a.h_kv + kvh) * D;
    const bf16 *src = (const bf16 *)(ROLE == 0 ? kbuf : vbuf) + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) kvf[kt][c] = kvalid[kt] ? ld_bf16x8(src + 16 * c + 8 * g) : zero_bf16x8();
  }
  const RowReader<D> rd(lane);
  const TrReader<D> tr(lane);
  f32x16 acc[ND][KT];   // dV^T (role 0) or dK^T (role 1): [head dim][keys]
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[dt][kt] = zero_f32x16();
  const int pofs = kw * (2 * KT * 4 * 64);   // this wave pair's slot in a P buffer
  auto pidx = [&](int h2, int kt, int s4) { return pofs + ((h2 * KT + kt) * 4 + s4) * 64 + lane; };

  // This workgroup's tiles t = 0 .. n - 1 are the key tile's tiles t0 + t: list
  // entry lb + (t0 + t) / G, head kvh * G + (t0 + t) % G.
  const int n = nt;
  const int q_stride = a.h_q * D;
  // Tile t's list entry record {q0, rows, full, q-tile} (a scalar load; t is
  // clamped to n - 1, so the entry stays inside this key tile's list).  Records
  // are fetched a full iteration before their tiles are used, which hides the
  // scalar load's latency.
  struct TileRef { int q0, nrows, full, h; };
  const u32x4 *lrec = reinterpret_cast<const u32x4 *>(a.lrec);
  auto fetch = [&](int t) { return ld_table(lrec, lb + (t0 + min(t, n - 1)) / G); };
  auto ref = [&](const u32x4 &r, int t) {
    TileRef x;
    x.q0 = (int)r[0];
    x.nrows = (int)r[1];
    x.full = (int)r[2];
    x.h = kvh * G + (t0 + min(t, n - 1)) % G;
    return x;
  };
  u32x4 rec1 = {0u, 0u, 0u, 0u}, rec2 = {0u, 0u, 0u, 0u};   // records of tiles i + 1 and i + 2
  // Loads of iteration i: Q(i + 2) and dO(i + 1), each with side rows.  Every
  // load is issued by the dK waves (4..7): a wave stalls at issue until the CU's
  // vector memory path accepts its loads, and the dK waves have the slack (their
  // iteration is shorter than the dV waves', which carry the exponentials).  The
  // side rows (one dword per lane) are issued at the start of the iteration.
  // Wave 4 fetches the Q tile's LSE into a register; lse_store() later puts the
  // exponent offset -LSE log2(e) into the side rows (FLT_MAX for a row without
  // keys, LSE = -inf, so that exp2(-inf + offset) is still 0).  Waves 6 and 7
  // fetch the rows' legal key bounds, wave 5 the dO tile's delta.  The tile loads
  // take 1 KB per instruction.
  float lse_reg = 0.f;
  // The side-row buffers start at the tile's first row (64-bit pointer
  // arithmetic), so their 32-bit record counts and offsets stay below 1 KB at
  // any row count.
  auto side_q = [&](const TileRef &r, int b) {
    const int rl = lane < r.nrows ? lane : r.nrows - 1;
    if (wave == 4) {
      lse_reg = a.lse[(int64_t)r.h * a.n_q + r.q0 + rl];
    } else if (wave == 6 || wave == 7) {
      dword_load_lds(a.rows + (int64_t)r.q0 * 4, r.nrows * 16, (rl * 4 + 2 * s + (wave - 6)) * 4,
                     &L.sq[b][wave - 5][0]);
    }
  };
  auto lse_store = [&](int b) {   // wave 4, once its loads have landed
    if (wave == 4) L.sq[b][0][lane] = fminf(-lse_reg * kLog2e, FLT_MAX);
  };
  auto side_d = [&](const TileRef &r, int b) {
    if (wave == 5) {
      const int rl = lane < r.nrows ? lane : r.nrows - 1;
      dword_load_lds(a.delta + (int64_t)r.h * a.n_q + r.q0, r.nrows * 4, rl * 4, L.sd[b]);
    }
  };
  auto tile_q = [&](const TileRef &r, int b) {
    if constexpr (ROLE == 1) {
      const int64_t off = (int64_t)r.q0 * q_stride + (int64_t)r.h * D;
      tile_load<D, NWR>(L.q[b], (const bf16 *)a.q + off, q_stride, r.nrows, wave - NWR, lane);
    }
  };
  auto tile_d = [&](const TileRef &r, int b) {
    if constexpr (ROLE == 1) {
      const int64_t off = (int64_t)r.q0 * q_stride + (int64_t)r.h * D;
      tile_load<D, NWR>(L.d[b], (const bf16 *)a.dout + off, q_stride, r.nrows, wave - NWR, lane);
    }
  };

  // dV waves, first half of P(t): S = Q K^T from Q buffer bq.  A masked tile
  // (masked pairs, or rows past the end) gets S = -inf on the illegal pairs, so
  // that their P is 0; this branch is rare and kept apart from the exponentials.
  f32x16 sc[2][KT];
  auto score_tile = [&](const TileRef &r, int bq) {
    const char *q_lds = L.q[bq];
    const float(*side)[BM] = L.sq[bq];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) sc[h2][kt] = zero_f32x16();
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 qa = rd(q_lds, h2, c);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sc[h2][kt] = mfma32(qa, kvf[kt][c], sc[h2][kt]);
      }
    if constexpr (KT == 1) pipeline_lds_mfma<2 * NC, 1, 4>();
    if (!r.full || r.nrows < BM) {
      keep_branch();
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int qb = 32 * h2 + 8 * s4 + 4 * g;       // rows qb .. qb + 3 of this lane
          const u32x4 lo4 = *reinterpret_cast<const u32x4 *>(&side[1][qb]);
          const u32x4 hi4 = *reinterpret_cast<const u32x4 *>(&side[2][qb]);
          const int left = r.nrows - qb;                  // rows qb + i with i < left exist
          // integer sign test (no per-element lane masks): the pair is illegal
          // iff one of left - 1 - i, key - lo, hi - 1 - key is negative; an
          // illegal score gets -inf added, a legal one +0
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int out = ((left - 1 - i) | (key[kt] - (int)lo4[i]) | ((int)hi4[i] - 1 - key[kt])) >> 31;
              sc[h2][kt][4 * s4 + i] += __int_as_float(out & (int)0xff800000u);
            }
        }
    }
  };
  // dV waves, second half: P = exp2(S scale log2(e) - LSE log2(e)) (the offset
  // from the side rows of Q buffer bq) into P buffer bp (fp32) and into pk (bf16
  // B operands for the dV MFMAs).
  bf16x8 pk[4][KT];   // [16-row chunk][key tile]
  auto exp_tile = [&](int bq, int bp) {
    f32x4 *pbuf = L.pb[bp];
    const float *nls = L.sq[bq][0];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 nl4 = *reinterpret_cast<const f32x4 *>(&nls[32 * h2 + 8 * s4 + 4 * g]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          f32x4 p4;
#pragma unroll
          for (int i = 0; i < 4; ++i) p4[i] = fast_exp2(fmaf(sc[h2][kt][4 * s4 + i], a.scale_log2, nl4[i]));
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[h2][kt][4 * s4 + i] = p4[i];
          pbuf[pidx(h2, kt, s4)] = p4;
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        pk[2 * h2][kt] = pack8(sc[h2][kt], 0);
        pk[2 * h2 + 1][kt] = pack8(sc[h2][kt], 8);
      }
    }
  };

  // iteration i with buffers fixed at compile time: K = i mod 6
  auto step = [&](auto kc, int i) {
    constexpr int K = decltype(kc)::value;
    wg_barrier();   // P(i) is in LDS; the buffers of iteration i - 1 are free
    const bool hq = i + 2 < n, hd = i + 1 < n;
    const TileRef r1 = ref(rec1, i + 1), r2 = ref(rec2, i + 2);
    const u32x4 rec3 = fetch(i + 3);
    if (hq) {
      side_q(r2, (K + 2) % 3);
      tile_q(r2, (K + 2) % 3);
    }
    if (hd) {
      side_d(r1, (K + 1) % 2);
      tile_d(r1, (K + 1) % 2);
    }
    if constexpr (ROLE == 0) {
      // S of tile i + 1 (of tile n - 1 again in the last iteration: computed, unused)
      bf16x8 pb[4][KT];
#pragma unroll
      for (int c16 = 0; c16 < 4; ++c16)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) pb[c16][kt] = pk[c16][kt];
      score_tile(r1, (K + 1) % 3);
      // dV^T += dO(i)^T P(i), independent of the exponentials of P(i + 1)
      const char *d_lds = L.d[K % 2];
#pragma unroll
      for (int c16 = 0; c16 < 4; ++c16)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const bf16x8 da = tr(d_lds, c16, dt);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) acc[dt][kt] = mfma32(da, pb[c16][kt], acc[dt][kt]);
        }
      exp_tile((K + 1) % 3, (K + 1) % 2);
      if constexpr (KT == 1) pipeline_lds_mfma<4 * ND, 2, 4>();
    } else {
      const char *d_lds = L.d[K % 2], *q_lds = L.q[K % 3];
      const f32x4 *pbuf = L.pb[K % 2];
      const float *dl = L.sd[K % 2];
      f32x16 dp[2][KT];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) dp[h2][kt] = zero_f32x16();
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 da = rd(d_lds, h2, c);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) dp[h2][kt] = mfma32(da, kvf[kt][c], dp[h2][kt]);
        }
      // dS = P o (dP - delta); dK^T += Q^T dS
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&dl[32 * h2 + 8 * s4 + 4 * g]);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const f32x4 p4 = pbuf[pidx(h2, kt, s4)];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) dp[h2][kt][4 * s4 + ii] = p4[ii] * (dp[h2][kt][4 * s4 + ii] - d4[ii]);
          }
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x8 db[KT];
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) db[kt] = pack8(dp[h2][kt], 8 * cc);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const bf16x8 qa = tr(q_lds, 2 * h2 + cc, dt);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) acc[dt][kt] = mfma32(qa, db[kt], acc[dt][kt]);
          }
        }
      }
      if constexpr (KT == 1) pipeline_lds_mfma<2 * NC + 4 * ND, 2, 4>();
    }
    wait_vmcnt<0>();
    if (i + 2 < n) lse_store((K + 2) % 3);
    wait_lgkm0();
    rec1 = rec2;
    rec2 = rec3;
  };

  if (n > 0) {
    // prologue: Q(0), Q(1), dO(0) and their side rows; P(0)
    const u32x4 rec0 = fetch(0);
    rec1 = fetch(1);
    rec2 = fetch(2);
    const TileRef r0 = ref(rec0, 0);
    side_q(r0, 0);
    tile_q(r0, 0);
    wait_vmcnt<0>();
    lse_store(0);
    side_d(r0, 0);
    tile_d(r0, 0);
    if (n > 1) {
      const TileRef r1 = ref(rec1, 1);
      side_q(r1, 1);
      tile_q(r1, 1);
    }
    wait_vmcnt<0>();
    if (n > 1) lse_store(1);
    wait_lgkm0();
    wg_barrier();
    if constexpr (ROLE == 0) {
      score_tile(r0, 0);
      exp_tile(0, 0);
    }
    wait_lgkm0();
  }
  for (int i = 0; i < n; i += 6) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < n) step(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 < n) step(std::integral_constant<int, 2>{}, i + 2);
    if (i + 3 < n) step(std::integral_constant<int, 3>{}, i + 3);
    if (i + 4 < n) step(std::integral_constant<int, 4>{}, i + 4);
    if (i + 5 < n) step(std::integral_constant<int, 5>{}, i + 5);
  }

  const float mul = ROLE == 0 ? 1.f : a.scale;
  if (a.split > 1) {
    // fp32 partial of this workgroup's share of the walk: dK at ro = 0, dV at 1
    const int ro = ROLE == 0 ? 1 : 0;
    const int64_t n_s = a.n_seg[s];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (!kvalid[kt]) continue;
      float *outp = a.part[s] + ((((int64_t)ro * a.split + chunk) * n_s + key[kt]) * a.h_kv + kvh) * D;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[dt][kt][4 * s4 + i] * mul;
          *reinterpret_cast<f32x4 *>(outp + 32 * dt + 8 * s4 + 4 * g) = v;
        }
    }
    return;
  }
  // the gradient buffer of this tile, found again from the wave's first key (no
  // register is kept live through the loop for it)
  void *dkbuf, *dvbuf;
  const int kw0 = SPLIT ? __builtin_amdgcn_readfirstlane(key[0]) : 0;
  const int kbase_end = kw0 - grad_buffer<SPLIT>(a, s, kw0, dkbuf, dvbuf);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    if (!kvalid[kt]) continue;
    bf16 *outp = (bf16 *)(ROLE == 0 ? dvbuf : dkbuf) + ((int64_t)(key[kt] - kbase_end) * a.h_kv + kvh) * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int d0 = 32 * dt + 8 * s4 + 4 * g;
        bf16x4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = (bf16)(acc[dt][kt][4 * s4 + i] * mul);
        *reinterpret_cast<bf16x4 *>(outp + d0) = b;
      }
  }
}

// Key tiles of 32 per wave of the dK/dV kernel (1: 8 waves, 2 per SIMD; 2: 4
// waves, one per SIMD with the whole register file).
constexpr int kDkdvKT = 1;
constexpr int kDkdvThreads = 2 * (4 / kDkdvKT) * 64;
static_assert(kDkdvThreads == BDATTN_DKDV_THREADS, "dK/dV workgroup size known to the scheduler");

// SPLIT: the clean segment sits in several buffers (a.sh, a.gsh).
template <int D, bool SPLIT>
__global__ __launch_bounds__(kDkdvThreads, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BM = BDATTN_BWD_BM;
  static_assert(BM == Tile<D>::ROWS, "query tile = one LDS tile");
  __shared__ __attribute__((aligned(1024))) char qs0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char qs1[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char qs2[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds1[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(16))) float sq0[3][BM];
  __shared__ __attribute__((aligned(16))) float sq1[3][BM];
  __shared__ __attribute__((aligned(16))) float sq2[3][BM];
  __shared__ __attribute__((aligned(16))) float sd0[BM];
  __shared__ __attribute__((aligned(16))) float sd1[BM];
  __shared__ f32x4 pb0[4 * 2 * 4 * 64];
  __shared__ f32x4 pb1[4 * 2 * 4 * 64];
  const DkdvLds<D> L = {{qs0, qs1, qs2}, {ds0, ds1}, {sq0, sq1, sq2}, {sd0, sd1}, {pb0, pb1}};
  const int wave = wave_id(), lane = threadIdx.x & 63;
  // workgroup = (key tile, share of its walk, KV head); consecutive workgroups
  // take different KV heads, so each XCD keeps to one KV head
  const int kvh = blockIdx.x % a.h_kv, rest = blockIdx.x / a.h_kv;
  const int kti = rest / a.split, chunk = rest % a.split;
  const int s = ld_table(a.ktiles, (int64_t)kti * 4), k0 = ld_table(a.ktiles, (int64_t)kti * 4 + 1);
  const int lb = ld_table(a.ktiles, (int64_t)kti * 4 + 2), le = ld_table(a.ktiles, (int64_t)kti * 4 + 3);
  const int total = (le - lb) * a.group;
  const int t0 = (int)((int64_t)total * chunk / a.split), t1 = (int)((int64_t)total * (chunk + 1) / a.split);
  if (wave < 4 / kDkdvKT) dkdv_role<D, kDkdvKT, 0, SPLIT>(a, s, k0, lb, t0, t1 - t0, chunk, kvh, wave, lane, L);
  else dkdv_role<D, kDkdvKT, 1, SPLIT>(a, s, k0, lb, t0, t1 - t0, chunk, kvh, wave, lane, L);
}

// Sum of the split dK/dV partials of one key segment, in chunk order (so the
// result does not depend on scheduling), to bf16: n4 groups of 4 elements per
// tensor, dK groups first, then dV.  The gradients go to n_buf buffers of
// per_buf groups each (the last holds the rest).
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float *part, int split, int64_t n4,
                                                          GradShardTable out, int n_buf, int64_t per_buf) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * n4) return;
  const int ro = i >= n4 ? 1 : 0;
  const int64_t e = i - ro * n4;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(part) + (int64_t)ro * split * n4 + e;
  f32x4 acc = src[0];
  for (int c = 1; c < split; ++c) acc += src[(int64_t)c * n4];
  bf16x4 b;
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = (bf16)acc[k];
  const int bi = n_buf > 1 ? (int)min(e / per_buf, (int64_t)n_buf - 1) : 0;
  reinterpret_cast<bf16x4 *>(ro ? out.dv[bi] : out.dk[bi])[e - bi * per_buf] = b;
}

// SPLIT: the clean segment sits in several buffers (a.sh).
template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * BDATTN_FWD_WAVES, 8 / BDATTN_FWD_WAVES) void dq_kernel(BwdArgs a) {
  constexpr int BN = BDATTN_FWD_BN;
  static_assert(BN == Tile<D>::ROWS, "key tile = one LDS tile");
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) char ks0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vs0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ks1[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vs1[Tile<D>::BYTES];

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, j = lane & 31, g = lane >> 5;
  const int item = blockIdx.x / a.h_q;
  const int pslot = blockIdx.x % a.h_q;
  const int h = (pslot % a.h_kv) * a.group + pslot / a.h_kv;
  const int kvh = h / a.group;
  const int32_t *it = a.items + (int64_t)item * 12;
  const int q0 = it[0], nrows = it[1];
  int lo_max[2], hi_min[2], base[2], nt[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int lmin = it[2 + 4 * s], lmax = it[3 + 4 * s], hmin = it[4 + 4 * s], hmax = it[5 + 4 * s];
    lo_max[s] = lmax;
    hi_min[s] = hmin;
    base[s] = lmin / BN * BN;
    nt[s] = hmax > lmin ? (hmax - base[s] + BN - 1) / BN : 0;
  }
  const int total = nt[0] + nt[1];
  if (total == 0) return;   // no key of this range: nothing to add

  const int rloc = wave * 32 + j;
  const bool valid = rloc < nrows;
  const int row = q0 + (valid ? rloc : 0);
  bf16x8 qf[NC], df[NC];
  {
    const int64_t off = ((int64_t)row * a.h_q + h) * D;
    const bf16 *qrow = (const bf16 *)a.q + off;
    const bf16 *drow = (const bf16 *)a.dout + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = valid ? ld_bf16x8(qrow + 16 * c + 8 * g) : zero_bf16x8();
      df[c] = valid ? ld_bf16x8(drow + 16 * c + 8 * g) : zero_bf16x8();
    }
  }
  int lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
  float l2 = INFINITY, dl = 0.f;
  if (valid) {
    const u32x4 rb = ld_u32x4(a.rows + (int64_t)row * 4);
    lo0 = (int)rb[0]; hi0 = (int)rb[1]; lo1 = (int)rb[2]; hi1 = (int)rb[3];
    const float l = a.lse[(int64_t)h * a.n_q + row];
    l2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dl = a.delta[(int64_t)h * a.n_q + row];
  }
  const RowReader<D> rd(lane);
  const TrReader<D> tr(lane);
  f32x16 dqa[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) dqa[dt] = zero_f32x16();

  const int kv_stride = a.h_kv * D;
  auto issue = [&](int t, char *kd, char *vd) {
    const int s = t < nt[0] ? 0 : 1;
    const int k0 = s == 0 ? base[0] + t * BN : base[1] + (t - nt[0]) * BN;
    // the buffer holding the key tile (a tile never straddles two)
    const void *kbuf, *vbuf;
    const int rb = seg_buffer<SPLIT>(a, s, k0, kbuf, vbuf);
    const int64_t off = (int64_t)rb * kv_stride + kvh * D;
    const int nv = a.n_seg[s] - k0;
    tile_load<D, BDATTN_FWD_WAVES>(kd, (const bf16 *)kbuf + off, kv_stride, nv, wave, lane);
    tile_load<D, BDATTN_FWD_WAVES>(vd, (const bf16 *)vbuf + off, kv_stride, nv, wave, lane);
  };
  auto compute = [&](int t, const char *k_lds, const char *v_lds) {
    const int s = t < nt[0] ? 0 : 1;
    const int k0 = s == 0 ? base[0] + t * BN : base[1] + (t - nt[0]) * BN;
    const bool full = lo_max[s] <= k0 && k0 + BN <= hi_min[s];
    const int lo = s ? lo1 : lo0, hi = s ? hi1 : hi0;
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = zero_f32x16();
      dp[kt] = zero_f32x16();
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = mfma32(rd(k_lds, kt, c), qf[c], sc[kt]);
        dp[kt] = mfma32(rd(v_lds, kt, c), df[c], dp[kt]);
      }
    pipeline_lds_mfma<4 * NC, 1, 8>();   // eight operands ahead (four measured 0.4-0.6% slower)
    if (!full) {
      keep_branch();
      // illegal pairs get S = -inf, hence P = 0.  Key k0 + 4 g + o (o an
      // immediate) is legal iff lo <= key < hi; the test is integer arithmetic
      // (sign of (o - lo) | (hi - 1 - o)) and adds -inf or +0, so no
      // per-element lane masks are formed.
      const int lo_r = lo - k0 - 4 * g, hi_r = hi - 1 - k0 - 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = kt * 32 + 8 * (r >> 2) + (r & 3);
          const int out = ((o - lo_r) | (hi_r - o)) >> 31;   // -1 if illegal, else 0
          sc[kt][r] += __int_as_float(out & (int)0xff800000u);
        }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(sc[kt][r], a.scale_log2, -l2));
        sc[kt][r] = pv * (dp[kt][r] - dl);     // dS^T
      }
#pragma unroll
    for (int c16 = 0; c16 < BN / 16; ++c16) {
      const bf16x8 db = pack8(sc[c16 >> 1], 8 * (c16 & 1));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) dqa[dt] = mfma32(tr(k_lds, c16, dt), db, dqa[dt]);
    }
  };

  // One barrier per key tile: after it, tile t has landed for every wave and
  // every wave is done with tile t - 1, whose buffer then takes tile t + 1.
  issue(0, ks0, vs0);
  for (int t = 0; t < total; t += 2) {
    wait_vmcnt<0>();
    wg_barrier();
    if (t + 1 < total) issue(t + 1, ks1, vs1);
    compute(t, ks0, vs0);
    wait_lgkm0();
    if (t + 1 < total) {
      wait_vmcnt<0>();
      wg_barrier();
      if (t + 2 < total) issue(t + 2, ks0, vs0);
      compute(t + 1, ks1, vs1);
      wait_lgkm0();
    }
  }

  if (!valid) return;
  float *dqp = a.dq + ((int64_t)row * a.h_q + h) * D;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int d0 = 32 * dt + 8 * s4 + 4 * g;
      f32x4 v = *reinterpret_cast<const f32x4 *>(dqp + d0);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaf(a.scale, dqa[dt][4 * s4 + i], v[i]);
      *reinterpret_cast<f32x4 *>(dqp + d0) = v;
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int32_t d, hipStream_t s, bool dkdv, bool dq) {
  const int64_t kblocks = dkdv ? (int64_t)a.n_kt * a.h_kv * a.split : 0;
  if (kblocks > 0) {
    const dim3 grid((unsigned)kblocks), block(kDkdvThreads);
    const bool split = a.sh.n > 1;
    if (d == 128) {
      if (split) hipLaunchKernelGGL((dkdv_kernel<128, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dkdv_kernel<128, false>), grid, block, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((dkdv_kernel<64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dkdv_kernel<64, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.split > 1) {
      for (int seg = 0; seg < 2; ++seg) {
        const int64_t n4 = (int64_t)a.n_seg[seg] * a.h_kv * d / 4;
        if (n4 == 0) continue;
        GradShardTable out{};
        int n_buf = 1;
        int64_t per_buf = n4;
        if (seg == 0) {
          out = a.gsh;
          n_buf = a.sh.n;
          if (n_buf > 1) per_buf = (int64_t)a.sh.len * a.h_kv * d / 4;
        } else {
          out.dk[0] = a.dk[1];
          out.dv[0] = a.dv[1];
        }
        hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)a.part[seg], a.split, n4, out, n_buf, per_buf);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  const int64_t qblocks = dq ? (int64_t)a.n_items * a.h_q : 0;
  if (qblocks > 0) {
    const dim3 grid((unsigned)qblocks), block(64 * BDATTN_FWD_WAVES);
    const bool split = a.sh.n > 1;
    if (d == 128) {
      if (split) hipLaunchKernelGGL((dq_kernel<128, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dq_kernel<128, false>), grid, block, 0, s, a);
    } else {
      if (split) hipLaunchKernelGGL((dq_kernel<64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((dq_kernel<64, false>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace bdattn
