// Forward partial of BDLM-masked core attention on gfx950.
//
// Core attention softmax(Q K^T) V ("Efficient Long-context Language Model
// Training by Core Attention Disaggregation", English abstract) restricted to
// the legal pairs of the BDLM mask, computed against one clean K/V range and,
// optionally, the rank's local corrupted K/V ("rit.work explainer of CSBP",
// section on why conventional context parallelism sends extra data).  Writes
// the range's partial O and its log-sum-exp, so that partials over disjoint
// ranges merge exactly.
//
// Layout of the work: one workgroup = 4 waves = 128 query rows of one q-head.
// Each wave owns 32 rows and computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16,
// so a lane holds one query (column) and 16 of its keys: the row max needs one
// cross-half exchange and the row sum stays in-lane.  The probabilities are fed
// straight from the C registers into O^T += V^T P^T as the B operand; V^T is
// read from a transposed copy whose keys are pre-permuted to match.
// Full key tiles skip the mask; partial tiles compare each key against the
// row's legal range.  The running max is only raised (and O, l rescaled) when
// it grows by more than 2^8, which keeps every probability below 256.
#include "common.h"
#include "kernels.h"

namespace bdattn {
namespace {

template <int D>
struct __attribute__((aligned(16))) FwdSmem {
  static constexpr int KS = D + 8;                 // K tile row stride (elements)
  static constexpr int VS = BDATTN_FWD_BN + 8;     // V^T tile row stride
  bf16 k[BDATTN_FWD_BN * KS];
  bf16 vt[D * VS];
};

template <int D>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  constexpr int BN = BDATTN_FWD_BN;
  constexpr int NC = D / 16;                 // 16-wide chunks of the head dim
  constexpr int ND = D / 32;                 // 32-wide tiles of the head dim
  constexpr int KCH = BN * D / 8 / 256;      // 16-byte chunks per thread, K tile
  constexpr int VCH = D * BN / 8 / 256;      // 16-byte chunks per thread, V^T tile
  using Sm = FwdSmem<D>;
  __shared__ Sm sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, g = lane >> 5;
  const int item = blockIdx.x / a.h_q;
  const int pslot = blockIdx.x % a.h_q;
  // consecutive workgroups land on different XCDs: give each XCD one KV head
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
    if (hmax > lmin) {
      base[s] = lmin / BN * BN;
      nt[s] = (hmax - base[s] + BN - 1) / BN;
    } else {
      base[s] = 0;
      nt[s] = 0;
    }
  }
  const int total = nt[0] + nt[1];

  const int rloc = wave * 32 + j;
  const bool valid = rloc < nrows;
  const int row = q0 + rloc;

  // Q as the B operand of S^T = K Q^T: lane (query j, group g) holds d = 16c + 8g .. +7.
  bf16x8 qf[NC];
  {
    const bf16 *qrow = (const bf16 *)a.q + ((int64_t)row * a.h_q + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = valid ? ld_bf16x8(qrow + 16 * c + 8 * g) : zero_bf16x8();
  }
  int lo[2] = {0, 0}, hi[2] = {0, 0};
  if (valid) {
    u32x4 rb = ld_u32x4(a.rows + (int64_t)row * 4);
    lo[0] = (int)rb[0]; hi[0] = (int)rb[1]; lo[1] = (int)rb[2]; hi[1] = (int)rb[3];
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) oacc[dt] = zero_f32x16();
  float m_used = -INFINITY;   // running max in log2 units, same in both halves of a query
  double l_sum = 0.0;         // this lane's share of the row sum

  u32x4 kreg[KCH], vreg[VCH];
  auto tile_seg = [&](int t) { return t < nt[0] ? 0 : 1; };
  auto tile_k0 = [&](int t) { return t < nt[0] ? base[0] + t * BN : base[1] + (t - nt[0]) * BN; };
  auto load_tile = [&](int t) {
    const int s = tile_seg(t), k0 = tile_k0(t);
    const bf16 *kb = (const bf16 *)a.k[s];
    const bf16 *vb = (const bf16 *)a.vt[s] + (int64_t)kvh * D * a.kpad[s] + k0;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), col = c % (D / 8), key = k0 + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = key < a.n_seg[s] ? ld_u32x4(kb + ((int64_t)key * a.h_kv + kvh) * D + col * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + 256 * i, r = c / (BN / 8), col = c % (BN / 8);
      vreg[i] = ld_u32x4(vb + (int64_t)r * a.kpad[s] + col * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), col = c % (D / 8);
      st_u32x4(&sm.k[r * Sm::KS + col * 8], kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + 256 * i, r = c / (BN / 8), col = c % (BN / 8);
      st_u32x4(&sm.vt[r * Sm::VS + col * 8], vreg[i]);
    }
  };

  if (total > 0) load_tile(0);
  for (int t = 0; t < total; ++t) {
    const int s = tile_seg(t), k0 = tile_k0(t);
    const bool full = lo_max[s] <= k0 && k0 + BN <= hi_min[s];
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < total) load_tile(t + 1);

    // S^T for two 32-key tiles: lane holds keys 8(r/4) + 4g + r%4 of query j.
    f32x16 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = zero_f32x16();
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sc[kt] = mfma32(ld_bf16x8(&sm.k[(kt * 32 + j) * Sm::KS + 16 * c + 8 * g]), qf[c], sc[kt]);
    }
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key < lo[s] || key >= hi[s]) sc[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mx2 = mx * a.scale_log2;
    if (__any(mx2 > m_used + 8.f)) {
      const float m_new = fmaxf(m_used, mx2);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_used - m_new);
      l_sum *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_used = m_new;
    }
    const float mb = (m_used == -INFINITY) ? 0.f : m_used;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(sc[kt][r], a.scale_log2, -mb));
        sc[kt][r] = pv;
        psum += pv;
      }
    l_sum += (double)psum;

    // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
    for (int c16 = 0; c16 < 4; ++c16) {
      const bf16x8 pb = pack8(sc[c16 >> 1], 8 * (c16 & 1));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        oacc[dt] = mfma32(ld_bf16x8(&sm.vt[(32 * dt + j) * Sm::VS + 16 * c16 + 8 * g]), pb, oacc[dt]);
    }
  }

  const double l_tot = l_sum + __shfl_xor(l_sum, 32);
  if (!valid) return;
  const bool has = l_tot > 0.0;
  const float inv = has ? (float)(1.0 / l_tot) : 0.f;
  if (g == 0) {
    const float lse = has ? (float)(((double)m_used + log2(l_tot)) * kLn2) : -INFINITY;
    a.lse[(int64_t)h * a.n_q + row] = lse;
  }
  const int64_t obase = ((int64_t)row * a.h_q + h) * D;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int d0 = 32 * dt + 8 * s4 + 4 * g;
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = oacc[dt][4 * s4 + i] * inv;
      if (a.o_f32) {
        *reinterpret_cast<f32x4 *>((float *)a.o + obase + d0) = v;
      } else {
        bf16x4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = (bf16)v[i];
        *reinterpret_cast<bf16x4 *>((bf16 *)a.o + obase + d0) = b;
      }
    }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int32_t d, hipStream_t s) {
  const int64_t blocks = (int64_t)a.n_items * a.h_q;
  if (blocks == 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(fwd_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fwd_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bdattn
