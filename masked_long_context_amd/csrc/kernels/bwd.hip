// Backward of BDLM-masked core attention on gfx950, for one K/V range.
//
// Gradients flow to the queries, the clean K/V range and the local corrupted
// K/V ("rit.work explainer of CSBP": conventional context parallelism returns
// the K/V gradients, CSBP returns only the clean ones and keeps the corrupted
// ones with their block).  With the MERGED log-sum-exp of every row, the
// probabilities of a range are exact, so per-range backwards add up to the
// unsharded one ("Block Parallelism For Efficient Distributed Long-Context
// Diffusion Language Model Training", English abstract: training semantics
// are preserved).
//
// One workgroup = 4 waves = 128 keys of one KV head (32 keys per wave).  It
// walks the list of query tiles (64 rows) that attend its keys, for each of the
// G q-heads of the group, and per tile computes with v_mfma_f32_32x32x16_bf16:
//   S = Q K^T, dP = dO V^T         (lane = key, K/V held in registers)
//   P = exp(S - LSE), dS = P o (dP - delta)
//   dV^T += dO^T P, dK^T += Q^T dS (P and dS feed the MFMA straight from C regs;
//                                    dO^T, Q^T come pre-transposed, rows permuted)
//   dQ += dS K                     (dS through LDS, K^T slice in registers, fp32
//                                    atomics into the accumulator)
// dK and dV are summed over the group in registers and written once.
#include "common.h"
#include "kernels.h"

namespace bdattn {
namespace {

template <int D>
struct __attribute__((aligned(16))) BwdSmem {
  static constexpr int BM = BDATTN_BWD_BM, BN = BDATTN_BWD_BN;
  static constexpr int RS = D + 8;     // row-major [BM][D] stride
  static constexpr int TS = BM + 8;    // transposed [D][BM] stride
  static constexpr int SS = BN + 8;    // dS [BM][BN] stride
  bf16 q[BM * RS];
  bf16 dout[BM * RS];
  bf16 qt[D * TS];
  bf16 dot[D * TS];
  bf16 ds[BM * SS];
  float lse2[BM];
  float delta[BM];
  int lo[BM];
  int hi[BM];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
  constexpr int BM = BDATTN_BWD_BM, BN = BDATTN_BWD_BN;
  constexpr int NC = D / 16, ND = D / 32;
  constexpr int NQT = (2 * ND) / 4;           // dQ output tiles per wave
  using Sm = BwdSmem<D>;
  __shared__ Sm sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, g = lane >> 5;
  const int kti = blockIdx.x / a.h_kv, kvh = blockIdx.x % a.h_kv;
  const int32_t *kd = a.ktiles + (int64_t)kti * 4;
  const int s = kd[0], k0 = kd[1], lb = kd[2], le = kd[3];
  const int key = k0 + wave * 32 + j;
  const bool kvalid = key < a.n_seg[s];

  // K and V as B operands (lane = key column, k = head dim).
  bf16x8 kf[NC], vf[NC];
  {
    const int64_t off = ((int64_t)key * a.h_kv + kvh) * D;
    const bf16 *kp = (const bf16 *)a.k[s] + off;
    const bf16 *vp = (const bf16 *)a.v[s] + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = kvalid ? ld_bf16x8(kp + 16 * c + 8 * g) : zero_bf16x8();
      vf[c] = kvalid ? ld_bf16x8(vp + 16 * c + 8 * g) : zero_bf16x8();
    }
  }
  // K^T slice as the B operand of dQ = dS K (lane = head-dim column, k = key).
  const int dq_dt = wave % ND;
  const int dq_t0 = (wave / ND) * NQT;
  bf16x8 ktf[BN / 16];
  {
    const bf16 *ktp = (const bf16 *)a.kt[s] + ((int64_t)kvh * D + dq_dt * 32 + j) * a.kpad[s] + k0;
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) ktf[c] = ld_bf16x8(ktp + 16 * c + 8 * g);
  }

  f32x16 dka[ND], dva[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    dka[dt] = zero_f32x16();
    dva[dt] = zero_f32x16();
  }

  for (int e = lb; e < le; ++e) {
    const int32_t ent = a.list[e];
    const bool full = ent < 0;
    const int qti = ent & 0x7fffffff;
    const int32_t *qd = a.bq + (int64_t)qti * 12;
    const int q0 = qd[0], nrows = qd[1];
    for (int hh = 0; hh < a.group; ++hh) {
      const int h = kvh * a.group + hh;
      __syncthreads();
      for (int c = tid; c < BM * D / 8; c += 256) {
        const int r = c / (D / 8), col = c % (D / 8);
        u32x4 z = {0u, 0u, 0u, 0u}, vq = z, vd = z;
        if (r < nrows) {
          const int64_t off = ((int64_t)(q0 + r) * a.h_q + h) * D + col * 8;
          vq = ld_u32x4((const bf16 *)a.q + off);
          vd = ld_u32x4((const bf16 *)a.dout + off);
        }
        st_u32x4(&sm.q[r * Sm::RS + col * 8], vq);
        st_u32x4(&sm.dout[r * Sm::RS + col * 8], vd);
      }
      {
        const int64_t slab = ((int64_t)qti * a.h_q + h) * D * BM;
        const bf16 *qts = (const bf16 *)a.qt + slab;
        const bf16 *dts = (const bf16 *)a.dot + slab;
        for (int c = tid; c < D * BM / 8; c += 256) {
          const int d = c / (BM / 8), col = c % (BM / 8);
          st_u32x4(&sm.qt[d * Sm::TS + col * 8], ld_u32x4(qts + d * BM + col * 8));
          st_u32x4(&sm.dot[d * Sm::TS + col * 8], ld_u32x4(dts + d * BM + col * 8));
        }
      }
      if (tid < BM) {
        const int r = tid;
        const bool v = r < nrows;
        const float l = v ? a.lse[(int64_t)h * a.n_q + q0 + r] : -INFINITY;
        sm.lse2[r] = (l == -INFINITY) ? INFINITY : l * kLog2e;   // P = 0 for rows without keys
        sm.delta[r] = v ? a.delta[(int64_t)h * a.n_q + q0 + r] : 0.f;
        if (!full) {
          sm.lo[r] = v ? a.rows[(int64_t)(q0 + r) * 4 + 2 * s] : 0;
          sm.hi[r] = v ? a.rows[(int64_t)(q0 + r) * 4 + 2 * s + 1] : 0;
        }
      }
      __syncthreads();

      f32x16 sc[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = zero_f32x16();
        dp[t] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sc[t] = mfma32(ld_bf16x8(&sm.q[(32 * t + j) * Sm::RS + 16 * c + 8 * g]), kf[c], sc[t]);
          dp[t] = mfma32(ld_bf16x8(&sm.dout[(32 * t + j) * Sm::RS + 16 * c + 8 * g]), vf[c], dp[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          float pv = fast_exp2(fmaf(sc[t][r], a.scale_log2, -sm.lse2[q]));
          if (!full && (key < sm.lo[q] || key >= sm.hi[q])) pv = 0.f;
          sc[t][r] = pv;
          dp[t][r] = pv * (dp[t][r] - sm.delta[q]);
        }
#pragma unroll
      for (int c2 = 0; c2 < BM / 16; ++c2) {
        const bf16x8 pb = pack8(sc[c2 >> 1], 8 * (c2 & 1));
        const bf16x8 db = pack8(dp[c2 >> 1], 8 * (c2 & 1));
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          dva[dt] = mfma32(ld_bf16x8(&sm.dot[(32 * dt + j) * Sm::TS + 16 * c2 + 8 * g]), pb, dva[dt]);
          dka[dt] = mfma32(ld_bf16x8(&sm.qt[(32 * dt + j) * Sm::TS + 16 * c2 + 8 * g]), db, dka[dt]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          sm.ds[q * Sm::SS + wave * 32 + j] = (bf16)dp[t][r];
        }
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < NQT; ++tt) {
        const int t = dq_t0 + tt;
        f32x16 acc = zero_f32x16();
#pragma unroll
        for (int c = 0; c < BN / 16; ++c)
          acc = mfma32(ld_bf16x8(&sm.ds[(32 * t + j) * Sm::SS + 16 * c + 8 * g]), ktf[c], acc);
        float *dqp = a.dq + ((int64_t)q0 * a.h_q + h) * D + dq_dt * 32 + j;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q < nrows) unsafeAtomicAdd(dqp + (int64_t)q * a.h_q * D, a.scale * acc[r]);
        }
      }
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

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int32_t d, hipStream_t s) {
  const int64_t blocks = (int64_t)a.n_kt * a.h_kv;
  if (blocks == 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(bwd_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bwd_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bdattn
