// Bandwidth-bound companions of the attention kernels on gfx950:
//   prepare    delta = rowsum(dO o O) (and a clear of the dQ accumulator)
//   merge      exact log-sum-exp merge of per-range partials
//   cast       fp32 -> bf16 (the dQ accumulator; the merged output)
#include "common.h"
#include "kernels.h"

namespace bdattn {
namespace {

// delta[h][r] = <dO[r][h], O[r][h]> (fp32), and the optional clear of the dQ
// accumulator.  D/8 threads per (row, head), each on 8 consecutive elements;
// the (row, head) pairs are taken in memory order, so a wave reads and writes
// one contiguous span.
template <int D>
__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs a) {
  constexpr int TPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gid / TPR;              // (row, head) in memory order
  const int sub = (int)(gid % TPR);
  const int64_t n_rh = (int64_t)a.n_q * a.h_q;
  float dot = 0.f;
  const bool valid = rh < n_rh;
  const int64_t off = rh * D + sub * 8;
  if (valid) {
    const bf16x8 db = ld_bf16x8((const bf16 *)a.dout + off);
    if (a.o_f32) {
      const f32x4 o0 = *reinterpret_cast<const f32x4 *>((const float *)a.o + off);
      const f32x4 o1 = *reinterpret_cast<const f32x4 *>((const float *)a.o + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += (float)db[e] * o0[e] + (float)db[e + 4] * o1[e];
    } else {
      const bf16x8 ob = ld_bf16x8((const bf16 *)a.o + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += (float)db[e] * (float)ob[e];
    }
    if (a.dq_zero) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4 *>(a.dq_zero + off) = z;
      *reinterpret_cast<f32x4 *>(a.dq_zero + off + 4) = z;
    }
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, TPR);
  if (valid && sub == 0) {
    const int64_t r = rh / a.h_q;
    const int h = (int)(rh % a.h_q);
    a.delta[(int64_t)h * a.n_q + r] = dot;
  }
}

// Partial LSEs a merge workgroup stages in LDS (more partials read them from
// global memory).
constexpr int kMergeStage = 64;

// D/4 lanes per (row, head); each lane merges 4 consecutive elements.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int n_parts, const void *op, int parts_f32,
                                                    const float *lp, int64_t n_rows, int h, void *oo,
                                                    int out_f32, float *lo) {
  constexpr int LPR = D / 4;
  constexpr int PAIRS = 256 / LPR;   // (row, head) pairs of the workgroup
  __shared__ float sl[kMergeStage][PAIRS];
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gid / LPR;
  const int sub = (int)(gid % LPR);
  const int pair = threadIdx.x / LPR;
  const int64_t n_rh = n_rows * h;
  const int64_t lstride = (int64_t)h * n_rows;
  // the workgroup's partial LSEs, read once into LDS
  const bool staged = n_parts <= kMergeStage;
  if (staged) {
    for (int i = threadIdx.x; i < n_parts * PAIRS; i += 256) {
      const int s = i / PAIRS, pr = i % PAIRS;
      const int64_t r2 = (int64_t)blockIdx.x * PAIRS + pr;
      sl[s][pr] = r2 < n_rh ? lp[s * lstride + (r2 % h) * n_rows + r2 / h] : -INFINITY;
    }
    __syncthreads();
  }
  if (rh >= n_rh) return;
  const int64_t n = rh / h;
  const int hh = (int)(rh % h);
  const int64_t lidx = (int64_t)hh * n_rows + n;
  auto lse_of = [&](int s) { return staged ? sl[s][pair] : lp[s * lstride + lidx]; };
  float m = -INFINITY;
  for (int s = 0; s < n_parts; ++s) m = fmaxf(m, lse_of(s));
  const int64_t oidx = rh * D + 4 * sub;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
    for (int s = 0; s < n_parts; ++s) tot += expf(lse_of(s) - m);
    lse = m + logf(tot);
    const int64_t ostride = n_rows * h * D;
    auto part = [&](int s) {
      f32x4 v;
      if (parts_f32) {
        v = *reinterpret_cast<const f32x4 *>((const float *)op + s * ostride + oidx);
      } else {
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>((const bf16 *)op + s * ostride + oidx);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (float)b[i];
      }
      return v;
    };
    // Partials in groups of four: the group's weights first, then its loads, all
    // issued before any is used, so that each lane keeps up to four loads in
    // flight.  A partial of weight 0 (LSE = -inf, or negligible) is not loaded:
    // its lanes are masked off and move no data.
    constexpr int U = 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + U <= n_parts; s += U) {
      float c[U];
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = expf(lse_of(s + u) - lse);
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = c[u] != 0.f ? part(s + u) : zero;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(c[u], v[u][i], acc[i]);
    }
    for (; s < n_parts; ++s) {
      const float c = expf(lse_of(s) - lse);
      const f32x4 v = c != 0.f ? part(s) : zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(c, v[i], acc[i]);
    }
  }
  if (out_f32) {
    *reinterpret_cast<f32x4 *>((float *)oo + oidx) = acc;
  } else {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (bf16)acc[i];
    *reinterpret_cast<bf16x4 *>((bf16 *)oo + oidx) = b;
  }
  if (sub == 0) lo[lidx] = lse;
}

// Round to nearest even, 8 elements per lane.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float *acc, bf16 *out, int64_t n) {
  const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i8 + 8 <= n) {
    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(acc + i8);
    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(acc + i8 + 4);
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = (bf16)a0[e];
      b[e + 4] = (bf16)a1[e];
    }
    *reinterpret_cast<bf16x8 *>(out + i8) = b;
  } else {
    for (int64_t i = i8; i < n; ++i) out[i] = (bf16)acc[i];
  }
}

}  // namespace

hipError_t launch_prepare(const PrepArgs &a, int32_t d, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const int64_t threads = (int64_t)a.n_q * a.h_q * (d / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (d == 128) hipLaunchKernelGGL(prepare_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(prepare_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(int32_t n_parts, const void *o_parts, bool parts_f32, const float *lse_parts,
                        int64_t n_rows, int32_t h, int32_t d, void *o_out, bool out_f32, float *lse_out,
                        hipStream_t s) {
  const int64_t threads = n_rows * h * (d / 4);
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(blocks), dim3(256), 0, s, n_parts, o_parts, parts_f32 ? 1 : 0,
                       lse_parts, n_rows, h, o_out, out_f32 ? 1 : 0, lse_out);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(blocks), dim3(256), 0, s, n_parts, o_parts, parts_f32 ? 1 : 0,
                       lse_parts, n_rows, h, o_out, out_f32 ? 1 : 0, lse_out);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float *acc, void *out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 256 * 8 - 1) / (256 * 8));
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks), dim3(256), 0, s, acc, (bf16 *)out, n);
  return hipGetLastError();
}

}  // namespace bdattn
