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
//   dkdv_kernel (key-major): one workgroup = 128 keys of one KV head (32 per
//     wave).  It walks the query tiles (64 rows) that attend its keys, for every
//     q-head of the group; K and V sit in registers as MFMA B operands, Q and dO
//     stream through double-buffered LDS tiles.  S = Q K^T and dP = dO V^T put
//     one key per lane, so P and dS feed dV^T += dO^T P and dK^T += Q^T dS
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
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace bdattn {
namespace {

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BM = BDATTN_BWD_BM;
  static_assert(BM == Tile<D>::ROWS, "query tile = one LDS tile");
  constexpr int NC = D / 16, ND = D / 32;
  constexpr int VMN = 2 * Tile<D>::LOADS / BDATTN_BWD_WAVES + 1;   // Q, dO tiles + one side row
  __shared__ __attribute__((aligned(1024))) char qs0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds0[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char qs1[Tile<D>::BYTES];
  __shared__ __attribute__((aligned(1024))) char ds1[Tile<D>::BYTES];
  // per query row of the tile: lse, delta, legal key range lo, hi
  __shared__ __attribute__((aligned(16))) float side0[4][BM];
  __shared__ __attribute__((aligned(16))) float side1[4][BM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, g = lane >> 5;
  const int kti = blockIdx.x / a.h_kv, kvh = blockIdx.x % a.h_kv;
  const int32_t *kd = a.ktiles + (int64_t)kti * 4;
  const int s = kd[0], k0 = kd[1], lb = kd[2], le = kd[3];
  const int key = k0 + wave * 32 + j;
  const bool kvalid = key < a.n_seg[s];
  const int G = a.group;

  // K and V as B operands (lane = key column, k = head dim).
  bf16x8 kf[NC], vf[NC];
  {
    const int64_t off = ((int64_t)(kvalid ? key : 0) * a.h_kv + kvh) * D;
    const bf16 *kp = (const bf16 *)a.k[s] + off;
    const bf16 *vp = (const bf16 *)a.v[s] + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = kvalid ? ld_bf16x8(kp + 16 * c + 8 * g) : zero_bf16x8();
      vf[c] = kvalid ? ld_bf16x8(vp + 16 * c + 8 * g) : zero_bf16x8();
    }
  }
  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    dka[dt] = zero_f32x16();
    dva[dt] = zero_f32x16();
  }

  const int n_iter = (le - lb) * G;
  const int64_t q_stride = (int64_t)a.h_q * D;
  auto issue = [&](int it, char *qd, char *dd, float (*side)[BM]) {
    const int e = lb + it / G, h = kvh * G + it % G;
    const int qti = a.list[e] & 0x7fffffff;
    const int q0 = a.bq[(int64_t)qti * 12], nrows = a.bq[(int64_t)qti * 12 + 1];
    const int64_t off = (int64_t)q0 * q_stride + (int64_t)h * D;
    tile_load<D, BDATTN_BWD_WAVES>(qd, (const bf16 *)a.q + off, q_stride, nrows, wave, lane);
    tile_load<D, BDATTN_BWD_WAVES>(dd, (const bf16 *)a.dout + off, q_stride, nrows, wave, lane);
    const int r = q0 + (lane < nrows ? lane : nrows - 1);
    const void *src;
    if (wave == 0) src = a.lse + (int64_t)h * a.n_q + r;
    else if (wave == 1) src = a.delta + (int64_t)h * a.n_q + r;
    else src = a.rows + (int64_t)r * 4 + 2 * s + (wave - 2);
    __builtin_amdgcn_global_load_lds(src, BD_LDS(&side[wave][0]), 4, 0, 0);
  };
  auto compute = [&](int it, const char *q_lds, const char *d_lds, const float (*side)[BM]) {
    const int e = lb + it / G;
    const int ent = a.list[e];
    const int qti = ent & 0x7fffffff;
    const int nrows = a.bq[(int64_t)qti * 12 + 1];
    const bool masked = ent >= 0 || nrows < BM;   // partial key range, or a ragged query tile
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 sc = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sc = mfma32(tile_row8<D>(q_lds, 32 * t + j, 16 * c + 8 * g), kf[c], sc);
        dp = mfma32(tile_row8<D>(d_lds, 32 * t + j, 16 * c + 8 * g), vf[c], dp);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int qb = 32 * t + 8 * s4 + 4 * g;          // rows qb .. qb + 3 of this lane
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&side[0][qb]);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&side[1][qb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * s4 + i;
          const float l2 = l4[i] == -INFINITY ? INFINITY : l4[i] * kLog2e;   // P = 0 for rows without keys
          float pv = fast_exp2(fmaf(sc[r], a.scale_log2, -l2));
          if (masked) {
            const int q = qb + i;
            const int lo = __float_as_int(side[2][q]), hi = __float_as_int(side[3][q]);
            if (q >= nrows || key < lo || key >= hi) pv = 0.f;
          }
          sc[r] = pv;
          dp[r] = pv * (dp[r] - d4[i]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c2 = 2 * t + cc;
        const bf16x8 pb = pack8(sc, 8 * cc);
        const bf16x8 db = pack8(dp, 8 * cc);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          dva[dt] = mfma32(tile_tr8<D>(d_lds, c2, dt, lane), pb, dva[dt]);
          dka[dt] = mfma32(tile_tr8<D>(q_lds, c2, dt, lane), db, dka[dt]);
        }
      }
    }
  };

  if (n_iter > 0) issue(0, qs0, ds0, side0);
  for (int it = 0; it < n_iter; it += 2) {
    if (it + 1 < n_iter) {
      issue(it + 1, qs1, ds1, side1);
      wait_vmcnt<VMN>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    compute(it, qs0, ds0, side0);
    wait_lgkm0();
    wg_barrier();
    if (it + 1 < n_iter) {
      if (it + 2 < n_iter) {
        issue(it + 2, qs0, ds0, side0);
        wait_vmcnt<VMN>();
      } else {
        wait_vmcnt<0>();
      }
      wg_barrier();
      compute(it + 1, qs1, ds1, side1);
      wait_lgkm0();
      wg_barrier();
    }
  }

  if (!kvalid) return;
  const int64_t obase = ((int64_t)key * a.h_kv + kvh) * D;
  bf16 *dkp = (bf16 *)a.dk[s] + obase;
  bf16 *dvp = (bf16 *)a.dv[s] + obase;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int d0 = 32 * dt + 8 * s4 + 4 * g;
      bf16x4 bk, bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bk[i] = (bf16)(dka[dt][4 * s4 + i] * a.scale);
        bv[i] = (bf16)dva[dt][4 * s4 + i];
      }
      *reinterpret_cast<bf16x4 *>(dkp + d0) = bk;
      *reinterpret_cast<bf16x4 *>(dvp + d0) = bv;
    }
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, g = lane >> 5;
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
  f32x16 dqa[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) dqa[dt] = zero_f32x16();

  const int64_t kv_stride = (int64_t)a.h_kv * D;
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
        sc[kt] = mfma32(tile_row8<D>(k_lds, kt * 32 + j, 16 * c + 8 * g), qf[c], sc[kt]);
        dp[kt] = mfma32(tile_row8<D>(v_lds, kt * 32 + j, 16 * c + 8 * g), df[c], dp[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(fmaf(sc[kt][r], a.scale_log2, -l2));
        if (!full) {
          const int key = k0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key < lo || key >= hi) pv = 0.f;
        }
        sc[kt][r] = pv * (dp[kt][r] - dl);     // dS^T
      }
#pragma unroll
    for (int c16 = 0; c16 < BN / 16; ++c16) {
      const bf16x8 db = pack8(sc[c16 >> 1], 8 * (c16 & 1));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) dqa[dt] = mfma32(tile_tr8<D>(k_lds, c16, dt, lane), db, dqa[dt]);
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

hipError_t launch_bwd(const BwdArgs &a, int32_t d, hipStream_t s) {
  const int64_t kblocks = (int64_t)a.n_kt * a.h_kv;
  if (kblocks > 0) {
    if (d == 128) hipLaunchKernelGGL(dkdv_kernel<128>, dim3((unsigned)kblocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dkdv_kernel<64>, dim3((unsigned)kblocks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t qblocks = (int64_t)a.n_items * a.h_q;
  if (qblocks > 0) {
    if (d == 128) hipLaunchKernelGGL(dq_kernel<128>, dim3((unsigned)qblocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dq_kernel<64>, dim3((unsigned)qblocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bdattn
