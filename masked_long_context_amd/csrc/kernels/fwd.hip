// Forward partial of BDLM-masked core attention on gfx950.
//
// Core attention softmax(Q K^T) V ("Efficient Long-context Language Model
// Training by Core Attention Disaggregation", English abstract) restricted to
// the legal pairs of the BDLM mask, against one clean K/V range and,
// optionally, the rank's local corrupted K/V ("rit.work explainer of CSBP",
// section on why conventional context parallelism sends extra data).  Writes
// the range's partial O and its log-sum-exp, so that partials over disjoint
// ranges merge exactly.
//
// One workgroup = BDATTN_FWD_WAVES waves (32 query rows each) of one q-head;
// every key tile it loads serves all its waves.  S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16) puts one query per lane and 16 of its keys in the
// lane's C registers: the row max needs one exchange across the wave halves and
// the row sum stays in-lane.  The probabilities go straight from the C
// registers into O^T += V^T P^T as the B operand; V^T comes from transpose reads
// of the row-major V tile.  K and V stream through two LDS buffers filled by
// direct global->LDS loads while the previous tile computes.
// Full key tiles skip the mask; partial tiles compare each key with the row's
// legal range.  The running max is only raised (rescaling O and l) when it grows
// by more than 2^8, which keeps every probability below 256.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace bdattn {
namespace {

// 64-row LDS tiles of K (and of V) per key step of the forward.
constexpr int kFwdTiles = BDATTN_FWD_STEP / 64;
static_assert(kFwdTiles * 64 == BDATTN_FWD_STEP, "forward step = whole LDS tiles");

// SPLIT: the clean segment sits in several buffers (a.sh).
template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * BDATTN_FWD_WAVES, 8 / BDATTN_FWD_WAVES) void fwd_kernel(FwdArgs a) {
  constexpr int KB = kFwdTiles;               // 64-row LDS tiles per key step
  constexpr int BN = KB * Tile<D>::ROWS;       // keys per step
  constexpr int TB = Tile<D>::BYTES;
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) char ks0[KB * TB];
  __shared__ __attribute__((aligned(1024))) char vs0[KB * TB];
  __shared__ __attribute__((aligned(1024))) char ks1[KB * TB];
  __shared__ __attribute__((aligned(1024))) char vs1[KB * TB];

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, j = lane & 31, g = lane >> 5;
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
    base[s] = lmin / BN * BN;
    nt[s] = hmax > lmin ? (hmax - base[s] + BN - 1) / BN : 0;
  }
  const int total = nt[0] + nt[1];

  const int rloc = wave * 32 + j;
  const bool valid = rloc < nrows;
  const int row = q0 + (valid ? rloc : 0);

  // Q as the B operand of S^T = K Q^T: lane (query j, half g) holds d = 16c + 8g .. +7.
  bf16x8 qf[NC];
  {
    const bf16 *qrow = (const bf16 *)a.q + ((int64_t)row * a.h_q + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = valid ? ld_bf16x8(qrow + 16 * c + 8 * g) : zero_bf16x8();
  }
  int lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
  if (valid) {
    const u32x4 rb = ld_u32x4(a.rows + (int64_t)row * 4);
    lo0 = (int)rb[0]; hi0 = (int)rb[1]; lo1 = (int)rb[2]; hi1 = (int)rb[3];
  }

  const RowReader<D> rd(lane);
  const TrReader<D> tr(lane);
  f32x16 oacc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) oacc[dt] = zero_f32x16();
  float m_used = -INFINITY;   // running max in log2 units, equal in both halves of a query
  double l_sum = 0.0;         // this lane's share of the row sum

  const int kv_stride = a.h_kv * D;
  auto issue = [&](int t, char *kd, char *vd) {
    const int s = t < nt[0] ? 0 : 1;
    const int k0 = s == 0 ? base[0] + t * BN : base[1] + (t - nt[0]) * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // a step starts below the segment's end; a later tile of it may not: its
      // rows then all re-read the last row (and are masked, the step not being full)
      int r0 = k0 + kb * Tile<D>::ROWS, nv = a.n_seg[s] - r0;
      if (nv < 1) {
        r0 = a.n_seg[s] - 1;
        nv = 1;
      }
      // the buffer holding the tile (a tile never straddles two)
      const void *kbuf, *vbuf;
      const int rb = seg_buffer<SPLIT>(a, s, r0, kbuf, vbuf);
      const int64_t off = (int64_t)rb * kv_stride + kvh * D;
      tile_load<D, BDATTN_FWD_WAVES>(kd + kb * TB, (const bf16 *)kbuf + off, kv_stride, nv, wave, lane);
      tile_load<D, BDATTN_FWD_WAVES>(vd + kb * TB, (const bf16 *)vbuf + off, kv_stride, nv, wave, lane);
    }
  };
  auto compute = [&](int t, const char *kt_lds, const char *vt_lds) {
    const int s = t < nt[0] ? 0 : 1;
    const int k0 = s == 0 ? base[0] + t * BN : base[1] + (t - nt[0]) * BN;
    const bool full = lo_max[s] <= k0 && k0 + BN <= hi_min[s];
    const int lo = s ? lo1 : lo0, hi = s ? hi1 : hi0;
    constexpr int NKT = BN / 32;   // 32-key column tiles of the step
    f32x16 sc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) sc[kt] = zero_f32x16();
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) sc[kt] = mfma32(rd(kt_lds + (kt >> 1) * TB, kt & 1, c), qf[c], sc[kt]);
    pipeline_lds_mfma<NKT * NC, 1, 8>();   // eight K operands ahead (four measured 0.3-0.5% slower)
    if (!full) {
      keep_branch();
      // key k0 + 4 g + o (o an immediate) is legal iff lo <= key < hi.  The
      // test is integer arithmetic (sign of (o - lo) | (hi - 1 - o)) and adds
      // -inf to an illegal score, so no per-element lane masks are formed.
      const int lo_r = lo - k0 - 4 * g, hi_r = hi - 1 - k0 - 4 * g;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = kt * 32 + 8 * (r >> 2) + (r & 3);
          const int out = ((o - lo_r) | (hi_r - o)) >> 31;       // -1 if illegal, else 0
          sc[kt][r] += __int_as_float(out & (int)0xff800000u);     // -inf or +0
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][r]);
    {
      // the other half of the query's keys sits 32 lanes away: v_permlane32_swap
      // of a register with itself gives every lane both halves' values (a VALU
      // op, where a shuffle would go through the LDS crossbar)
      const auto hv = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(hv[0]), __uint_as_float(hv[1]));
    }
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
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(sc[kt][r], a.scale_log2, -mb));
        sc[kt][r] = pv;
        psum += pv;
      }
    l_sum += (double)psum;
#pragma unroll
    for (int c16 = 0; c16 < BN / 16; ++c16) {
      const bf16x8 pb = pack8(sc[c16 >> 1], 8 * (c16 & 1));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) oacc[dt] = mfma32(tr(vt_lds + (c16 >> 2) * TB, c16 & 3, dt), pb, oacc[dt]);
    }
  };

  // One barrier per key tile: after it, tile t has landed for every wave and
  // every wave is done with tile t - 1, whose buffer then takes tile t + 1.
  if (total > 0) issue(0, ks0, vs0);
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
  const dim3 grid((unsigned)blocks), block(64 * BDATTN_FWD_WAVES);
  const bool split = a.sh.n > 1;
  if (d == 128) {
    if (split) hipLaunchKernelGGL((fwd_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (split) hipLaunchKernelGGL((fwd_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bdattn
