// Bandwidth-bound companions of the attention kernels on gfx950:
//   transpose  K or V [n][h_kv][d] -> [h_kv][d][kpad] (MFMA operand copies)
//   prepare    delta = rowsum(dO o O) and transposed Q / dO slabs per query tile
//   merge      exact log-sum-exp merge of per-range partials
//   finalize   fp32 dQ accumulator -> bf16
#include "common.h"
#include "kernels.h"

namespace bdattn {
namespace {

// One block = 64 keys of one KV head.  permute: store each 16-key chunk in the
// order a 32x32 MFMA's C registers hold it (see perm16).
template <int D>
__global__ __launch_bounds__(256) void transpose_kernel(const bf16 *x, int64_t n, int h_kv, int64_t kpad,
                                                         int permute, bf16 *out) {
  __shared__ __attribute__((aligned(16))) bf16 tile[D][64 + 8];
  const int tid = threadIdx.x;
  const int kvh = blockIdx.y;
  const int64_t key0 = (int64_t)blockIdx.x * 64;
  for (int c = tid; c < 64 * D / 8; c += 256) {
    const int r = c / (D / 8), col = c % (D / 8);
    const int64_t key = key0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < n) v = ld_u32x4(x + (key * h_kv + kvh) * D + col * 8);
    const bf16x8 b = __builtin_bit_cast(bf16x8, v);
    const int pos = permute ? ((r & ~15) | perm16(r & 15)) : r;
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[col * 8 + e][pos] = b[e];
  }
  __syncthreads();
  for (int c = tid; c < D * 8; c += 256) {
    const int d = c / 8, col = c % 8;
    st_u32x4(out + ((int64_t)kvh * D + d) * kpad + key0 + col * 8, ld_u32x4(&tile[d][col * 8]));
  }
}

// One block = one backward query tile (BWD_BM rows) of one q-head.
template <int D>
__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs a) {
  constexpr int BM = BDATTN_BWD_BM;
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) bf16 tq[D][BM + 8];
  __shared__ __attribute__((aligned(16))) bf16 tdo[D][BM + 8];
  __shared__ float part[BM][CPR + 1];
  const int tid = threadIdx.x;
  const int qti = blockIdx.x, h = blockIdx.y;
  const int q0 = a.bq[(int64_t)qti * 12], nrows = a.bq[(int64_t)qti * 12 + 1];
  for (int c = tid; c < BM * CPR; c += 256) {
    const int r = c / CPR, col = c % CPR;
    u32x4 vq = {0u, 0u, 0u, 0u}, vd = vq;
    float dot = 0.f;
    if (r < nrows) {
      const int64_t off = ((int64_t)(q0 + r) * a.h_q + h) * D + col * 8;
      vq = ld_u32x4((const bf16 *)a.q + off);
      vd = ld_u32x4((const bf16 *)a.dout + off);
      const bf16x8 db = __builtin_bit_cast(bf16x8, vd);
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
    }
    part[r][col] = dot;
    const bf16x8 qb = __builtin_bit_cast(bf16x8, vq);
    const bf16x8 db = __builtin_bit_cast(bf16x8, vd);
    const int pos = (r & ~15) | perm16(r & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tq[col * 8 + e][pos] = qb[e];
      tdo[col * 8 + e][pos] = db[e];
    }
  }
  __syncthreads();
  if (tid < nrows) {
    float acc = 0.f;
#pragma unroll
    for (int col = 0; col < CPR; ++col) acc += part[tid][col];
    a.delta[(int64_t)h * a.n_q + q0 + tid] = acc;
  }
  if (a.dq_zero) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int c = tid; c < nrows * (D / 4); c += 256) {
      const int r = c / (D / 4), col = c % (D / 4);
      *reinterpret_cast<f32x4 *>(a.dq_zero + ((int64_t)(q0 + r) * a.h_q + h) * D + col * 4) = z;
    }
  }
  const int64_t slab = ((int64_t)qti * a.h_q + h) * D * BM;
  for (int c = tid; c < D * BM / 8; c += 256) {
    const int d = c / (BM / 8), col = c % (BM / 8);
    st_u32x4((bf16 *)a.qt + slab + d * BM + col * 8, ld_u32x4(&tq[d][col * 8]));
    st_u32x4((bf16 *)a.dot + slab + d * BM + col * 8, ld_u32x4(&tdo[d][col * 8]));
  }
}

// D/4 lanes per (row, head); each lane merges 4 consecutive elements.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int n_parts, const void *op, int parts_f32,
                                                    const float *lp, int64_t n_rows, int h, void *oo,
                                                    int out_f32, float *lo) {
  constexpr int LPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gid / LPR;
  const int sub = (int)(gid % LPR);
  if (rh >= n_rows * h) return;
  const int64_t n = rh / h;
  const int hh = (int)(rh % h);
  const int64_t lstride = (int64_t)h * n_rows;
  const int64_t lidx = (int64_t)hh * n_rows + n;
  float m = -INFINITY;
  for (int s = 0; s < n_parts; ++s) m = fmaxf(m, lp[s * lstride + lidx]);
  const int64_t oidx = rh * D + 4 * sub;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
    for (int s = 0; s < n_parts; ++s) tot += expf(lp[s * lstride + lidx] - m);
    lse = m + logf(tot);
    const int64_t ostride = n_rows * h * D;
    for (int s = 0; s < n_parts; ++s) {
      const float c = expf(lp[s * lstride + lidx] - lse);
      if (c == 0.f) continue;
      f32x4 v;
      if (parts_f32) {
        v = *reinterpret_cast<const f32x4 *>((const float *)op + s * ostride + oidx);
      } else {
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>((const bf16 *)op + s * ostride + oidx);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (float)b[i];
      }
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

__global__ __launch_bounds__(256) void dq_finalize_kernel(const float *acc, bf16 *out, int64_t n) {
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

hipError_t launch_transpose(const void *x, int64_t n, int32_t h_kv, int32_t d, int64_t kpad, bool permute,
                            void *out, hipStream_t s) {
  if (kpad == 0) return hipSuccess;
  dim3 grid((unsigned)(kpad / 64), (unsigned)h_kv);
  if (d == 128)
    hipLaunchKernelGGL(transpose_kernel<128>, grid, dim3(256), 0, s, (const bf16 *)x, n, h_kv, kpad,
                       permute ? 1 : 0, (bf16 *)out);
  else
    hipLaunchKernelGGL(transpose_kernel<64>, grid, dim3(256), 0, s, (const bf16 *)x, n, h_kv, kpad,
                       permute ? 1 : 0, (bf16 *)out);
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepArgs &a, int32_t d, hipStream_t s) {
  if (a.n_bq == 0) return hipSuccess;
  dim3 grid((unsigned)a.n_bq, (unsigned)a.h_q);
  if (d == 128) hipLaunchKernelGGL(prepare_kernel<128>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(prepare_kernel<64>, grid, dim3(256), 0, s, a);
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

hipError_t launch_dq_finalize(const float *acc, void *out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 256 * 8 - 1) / (256 * 8));
  hipLaunchKernelGGL(dq_finalize_kernel, dim3(blocks), dim3(256), 0, s, acc, (bf16 *)out, n);
  return hipGetLastError();
}

}  // namespace bdattn
