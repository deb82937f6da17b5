// bdattn_fwd_static: the forward of one clean K/V range for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  It runs the same kernel as bdattn_fwd;
// the plan's forward tables, which bdattn_fwd uploads into the caller's
// workspace, go into a file-scope device array instead, so the call takes no
// workspace and allocates nothing.
#include <hip/hip_runtime.h>

#include "capi_internal.h"

namespace {

using bdattn::abi::fail;

constexpr int64_t kScratchBytes = 8ll << 20;   // 8 MiB per GPU, held until the process ends
constexpr int kMaxDevices = 64;

// The forward tables of the last bdattn_fwd_static call on each GPU.  In host
// code this name is a host-side stand-in, not a device address: host code uses
// only the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The address of `scratch` on the current device, looked up on the first call there.
int scratch_here(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BDATTN_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BDATTN_EUNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(BDATTN_EHIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
    if (!ptr) return fail(BDATTN_EHIP, "hipGetSymbolAddress returned NULL");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return BDATTN_OK;
}

}  // namespace

extern "C" int bdattn_fwd_static(const bdattn_plan *pl, const void *q, const void *k_clean, const void *v_clean,
                                 const void *k_corr, const void *v_corr, void *o, int32_t o_dtype, float *lse,
                                 void *stream) {
  if (!pl) return fail(BDATTN_EINVAL, "plan is NULL");
  if (pl->p.kind != 0) return fail(BDATTN_EINVAL, "plan is a varlen plan; bdattn_fwd_static takes BDLM plans");
  int rc = bdattn::abi::check_fwd_args(pl, q, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse);
  if (rc != BDATTN_OK) return rc;
  const int64_t need = bdattn::abi::fwd_table_bytes(pl);
  if (need > kScratchBytes)
    return fail(BDATTN_EWORKSPACE, "the plan's forward tables need " + std::to_string(need) +
                                       " bytes, more than the 8 MiB static scratch (about 500K query rows)");
  if (pl->p.n_q == 0) return BDATTN_OK;
  void *tables = nullptr;
  rc = scratch_here(&tables);
  if (rc != BDATTN_OK) return rc;
  bdattn_plan *mp = const_cast<bdattn_plan *>(pl);
  {
    std::lock_guard<std::mutex> lk(mp->mu);
    mp->p.used = true;   // bdattn_plan_destroy then waits for the device before freeing the host image
  }
  hipStream_t s = (hipStream_t)stream;
  // every call overwrites the whole table prefix it reads: nothing is left to clear
  hipError_t e = hipMemcpyAsync(tables, pl->p.image.data(), need, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(BDATTN_EHIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
  return bdattn::abi::launch_fwd_on_tables(pl, tables, q, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse, s);
}
