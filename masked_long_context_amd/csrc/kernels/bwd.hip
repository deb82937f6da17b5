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
//     group; Q and dO stream through double-buffered LDS tiles.  Eight waves,
//     two per SIMD: four "dV waves" (32 keys each, K in registers) compute
//     S = Q K^T, P and dV^T += dO^T P; four "dK waves" on the same keys (V in
//     registers) compute dP = dO V^T, take P from the dV waves through LDS, and
//     form dS and dK^T += Q^T dS.  Each wave keeps one accumulator and one
//     operand set, so two waves fit every SIMD and one's exp/VALU work overlaps
//     the other's MFMAs; the MFMA work per pair is that of a fused kernel.  S
//     and dP put one key per lane, so P and dS feed the accumulating MFMAs
//     straight from the C registers (dO^T and Q^T come from transpose reads).
//     dK and dV are summed over the group in registers and written once.
//   dq_kernel (query-major, shaped like the forward): one workgroup = 128 rows
//     of one q-head.  S^T = K Q^T and dP^T = V dO^T put one query per lane (its
//     LSE and delta are scalars), and dQ^T += K^T dS^T takes dS^T from the C
//     registers and K^T from transpose reads of the K tile.  dQ is owned by one
//     workgroup per call: it is added to the fp32 accumulator without atomics.
// The split recomputes S and dP once more than a fused kernel, but removes the
// fp32 atomics a fused key-major kernel needs for dQ (about one per useful pair
// and head), which the L2 executes far slower than the MFMA work they replace.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace bdattn {
namespace {

// The loop of one dkdv role.  Both roles walk the same (query tile, head)
// sequence over the shared double-buffered Q/dO tiles and pass the same
// barriers; per tile:
//   phase A  role 0 (dV waves, hold K): S = Q K^T, P = exp(S - LSE) on the legal
//            pairs; P (fp32) goes to LDS in the C-register layout.
//            role 1 (dK waves, hold V): dP = dO V^T.
//   barrier
//   phase B  role 0: dV^T += dO^T P.
//            role 1: reads P back (same lane <-> key map), dS = P o (dP - delta),
//            dK^T += Q^T dS.
template <int D, int ROLE>
__device__ __forceinline__ void dkdv_role(const BwdArgs &a, int s, int k0, int lb, int le, int kvh,
                                          int wave, int lane, char *qs0, char *ds0, char *qs1, char *ds1,
                                          float (*side0)[BDATTN_BWD_BM], float (*side1)[BDATTN_BWD_BM],
                                          f32x4 *pbuf) {
  constexpr int BM = BDATTN_BWD_BM;
  constexpr int NW = 2 * BDATTN_BWD_WAVES;
  constexpr int NC = D / 16, ND = D / 32;
  constexpr int VMT = 2 * Tile<D>::LOADS / NW;   // tile loads per wave per iteration
  const int j = lane & 31, g = lane >> 5;
  const int kw = wave & 3;
  const int key = k0 + kw * 32 + j;
  const bool kvalid = key < a.n_seg[s];
  const int G = a.group;

  // K (dV waves) or V (dK waves) as the B operand (lane = key column, k = head dim).
  bf16x8 kvf[NC];
  {
    const int64_t off = ((int64_t)(kvalid ? key : 0) * a.h_kv + kvh) * D;
    const bf16 *src = (const bf16 *)(ROLE == 0 ? a.k[s] : a.v[s]) + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) kvf[c] = kvalid ? ld_bf16x8(src + 16 * c + 8 * g) : zero_bf16x8();
  }
  const RowReader<D> rd(lane);
  const TrReader<D> tr(lane);
  f32x16 acc[ND];   // dV^T (role 0) or dK^T (role 1): [head dim][32 keys]
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) acc[dt] = zero_f32x16();
  // this wave pair's P slot: [half][register quad][lane] of f32x4
  f32x4 *pslot = pbuf + kw * (2 * 4 * 64);

  const int n_iter = (le - lb) * G;
  const int q_stride = a.h_q * D;
  auto issue = [&](int it, char *qd, char *dd, float (*side)[BM]) {
    const int e = lb + it / G, h = kvh * G + it % G;
    const int qti = ld_table(a.list, e) & 0x7fffffff;
    const int q0 = ld_table(a.bq, (int64_t)qti * 12), nrows = ld_table(a.bq, (int64_t)qti * 12 + 1);
    const int64_t off = (int64_t)q0 * q_stride + (int64_t)h * D;
    tile_load<D, NW>(qd, (const bf16 *)a.q + off, q_stride, nrows, wave, lane);
    tile_load<D, NW>(dd, (const bf16 *)a.dout + off, q_stride, nrows, wave, lane);
    if constexpr (ROLE == 0) {   // waves 0..3 also fetch the side rows: lse, delta, lo, hi
      const int r = q0 + (lane < nrows ? lane : nrows - 1);
      const void *src;
      if (wave == 0) src = a.lse + (int64_t)h * a.n_q + r;
      else if (wave == 1) src = a.delta + (int64_t)h * a.n_q + r;
      else src = a.rows + (int64_t)r * 4 + 2 * s + (wave - 2);
      __builtin_amdgcn_global_load_lds(src, BD_LDS(&side[wave][0]), 4, 0, 0);
    }
  };
  // wait until this wave's loads of the current tile landed; the next tile's stay in flight
  auto wait_current = [&](bool next_issued) {
    if (!next_issued) wait_vmcnt<0>();
    else if constexpr (ROLE == 0) wait_vmcnt<VMT + 1>();
    else wait_vmcnt<VMT>();
  };

  // dV waves: P of one 32-row half.  MASKED: the tile holds masked pairs or rows
  // past the end; each pair is checked against its row's legal key range (a row
  // without keys has LSE = -inf and gets P = 0).  Unmasked tiles only hold rows
  // that attend every key of the tile, whose merged LSE is finite.
  auto make_p = [&](auto masked_tag, int t, int nrows, const char *q_lds, const float (*side)[BM]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 sc = zero_f32x16();
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = mfma32(rd(q_lds, t, c), kvf[c], sc);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int qb = 32 * t + 8 * s4 + 4 * g;          // rows qb .. qb + 3 of this lane
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&side[0][qb]);
      f32x4 p4;
      if constexpr (MASKED) {
        const u32x4 lo4 = *reinterpret_cast<const u32x4 *>(&side[2][qb]);
        const u32x4 hi4 = *reinterpret_cast<const u32x4 *>(&side[3][qb]);
        const int left = nrows - qb;                     // rows qb + i with i < left exist
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(sc[4 * s4 + i], a.scale_log2, -l4[i] * kLog2e));
          const bool ok = (i < left) & (key >= (int)lo4[i]) & (key < (int)hi4[i]);
          p4[i] = ok ? pv : 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) p4[i] = fast_exp2(fmaf(sc[4 * s4 + i], a.scale_log2, -l4[i] * kLog2e));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * s4 + i] = p4[i];
      pslot[(t * 4 + s4) * 64 + lane] = p4;
    }
    return sc;
  };

  auto compute = [&](int it, const char *q_lds, const char *d_lds, const float (*side)[BM]) {
    if constexpr (ROLE == 0) {
      const int e = lb + it / G;
      const int ent = ld_table(a.list, e);
      const int nrows = ld_table(a.bq, (int64_t)(ent & 0x7fffffff) * 12 + 1);
      f32x16 p0, p1;
      if (ent >= 0 || nrows < BM) {   // partial key range, or a ragged query tile
        p0 = make_p(std::true_type{}, 0, nrows, q_lds, side);
        p1 = make_p(std::true_type{}, 1, nrows, q_lds, side);
      } else {
        p0 = make_p(std::false_type{}, 0, nrows, q_lds, side);
        p1 = make_p(std::false_type{}, 1, nrows, q_lds, side);
      }
      wait_lgkm0();
      wg_barrier();
      // dV^T += dO^T P
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 pb = pack8(t == 0 ? p0 : p1, 8 * cc);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(tr(d_lds, 2 * t + cc, dt), pb, acc[dt]);
        }
    } else {
      f32x16 dp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dp[t] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < NC; ++c) dp[t] = mfma32(rd(d_lds, t, c), kvf[c], dp[t]);
      }
      wait_lgkm0();
      wg_barrier();
      // dS = P o (dP - delta); dK^T += Q^T dS
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const f32x4 p4 = pslot[(t * 4 + s4) * 64 + lane];
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&side[1][32 * t + 8 * s4 + 4 * g]);
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[t][4 * s4 + i] = p4[i] * (dp[t][4 * s4 + i] - d4[i]);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 db = pack8(dp[t], 8 * cc);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(tr(q_lds, 2 * t + cc, dt), db, acc[dt]);
        }
      }
    }
  };

  if (n_iter > 0) issue(0, qs0, ds0, side0);
  for (int it = 0; it < n_iter; it += 2) {
    if (it + 1 < n_iter) issue(it + 1, qs1, ds1, side1);
    wait_current(it + 1 < n_iter);
    wg_barrier();
    compute(it, qs0, ds0, side0);
    wait_lgkm0();
    wg_barrier();
    if (it + 1 < n_iter) {
      if (it + 2 < n_iter) issue(it + 2, qs0, ds0, side0);
      wait_current(it + 2 < n_iter);
      wg_barrier();
      compute(it + 1, qs1, ds1, side1);
      wait_lgkm0();
      wg_barrier();
    }
  }

  if (!kvalid) return;
  const float mul = ROLE == 0 ? 1.f : a.scale;
  bf16 *outp = (bf16 *)(ROLE == 0 ? a.dv[s] : a.dk[s]) + ((int64_t)key * a.h_kv + kvh) * D;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int d0 = 32 * dt + 8 * s4 + 4 * g;
      bf16x4 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = (bf16)(acc[dt][4 * s4 + i] * mul);
      *reinterpret_cast<bf16x4 *>(outp + d0) = b;
    }
}

template <int D>
__global__ __launch_bounds__(2 * 256, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BM = BDATTN_BWD_BM;
  static_assert(BM == Tile<D>::ROWS, "query tile = one LDS tile");
  __shared__ __attribute__((aligned(1024))) char qs0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char qs1[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds1[Tile<D>::BYTES];
  // per query row of the tile: lse, delta, legal key range lo, hi
  __shared__ __attribute__((aligned(16))) float side0[4][BM];
  __shared__ __attribute__((aligned(16))) float side1[4][BM];
  // P of the current tile, handed from the dV waves to the dK waves
  __shared__ f32x4 pbuf[4 * 2 * 4 * 64];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int kti = blockIdx.x / a.h_kv, kvh = blockIdx.x % a.h_kv;
  const int s = ld_table(a.ktiles, (int64_t)kti * 4), k0 = ld_table(a.ktiles, (int64_t)kti * 4 + 1);
  const int lb = ld_table(a.ktiles, (int64_t)kti * 4 + 2), le = ld_table(a.ktiles, (int64_t)kti * 4 + 3);
  if (wave < 4) dkdv_role<D, 0>(a, s, k0, lb, le, kvh, wave, lane, qs0, ds0, qs1, ds1, side0, side1, pbuf);
  else dkdv_role<D, 1>(a, s, k0, lb, le, kvh, wave, lane, qs0, ds0, qs1, ds1, side0, side1, pbuf);
}

template <int D>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
  constexpr int BN = BDATTN_FWD_BN;
  static_assert(BN == Tile<D>::ROWS, "key tile = one LDS tile");
  constexpr int NC = D / 16, ND = D / 32;
  constexpr int VMN = 2 * Tile<D>::LOADS / BDATTN_FWD_WAVES;
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
    const int64_t off = (int64_t)k0 * kv_stride + kvh * D;
    const int nv = a.n_seg[s] - k0;
    tile_load<D, BDATTN_FWD_WAVES>(kd, (const bf16 *)a.k[s] + off, kv_stride, nv, wave, lane);
    tile_load<D, BDATTN_FWD_WAVES>(vd, (const bf16 *)a.v[s] + off, kv_stride, nv, wave, lane);
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
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sc[kt] = mfma32(rd(k_lds, kt, c), qf[c], sc[kt]);
        dp[kt] = mfma32(rd(v_lds, kt, c), df[c], dp[kt]);
      }
    }
    if (!full) {
      keep_branch();
      // illegal pairs get S = -inf, hence P = 0
      const int lo_r = lo - k0 - 4 * g, hi_r = hi - k0 - 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = kt * 32 + 8 * (r >> 2) + (r & 3);
          if (o < lo_r || o >= hi_r) sc[kt][r] = -INFINITY;
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

  issue(0, ks0, vs0);
  for (int t = 0; t < total; t += 2) {
    if (t + 1 < total) {
      issue(t + 1, ks1, vs1);
      wait_vmcnt<VMN>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    compute(t, ks0, vs0);
    wait_lgkm0();
    wg_barrier();
    if (t + 1 < total) {
      if (t + 2 < total) {
        issue(t + 2, ks0, vs0);
        wait_vmcnt<VMN>();
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier();
      compute(t + 1, ks1, vs1);
      wait_lgkm0();
      wg_barrier();
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
  const int64_t kblocks = dkdv ? (int64_t)a.n_kt * a.h_kv : 0;
  if (kblocks > 0) {
    if (d == 128) hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)kblocks), dim3(512), 0, s, a);
    else hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)kblocks), dim3(512), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t qblocks = dq ? (int64_t)a.n_items * a.h_q : 0;
  if (qblocks > 0) {
    if (d == 128) hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)qblocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)qblocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bdattn
