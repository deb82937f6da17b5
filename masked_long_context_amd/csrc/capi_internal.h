// Internals shared by the C ABI's source files (not part of the public header).
#pragma once
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <string>

#include "bdattn.h"
#include "plan.h"

struct bdattn_plan {
  bdattn::Plan p;
  std::mutex mu;   // guards the lazily made pinned copy of the tables and `used`
  // Workspace that holds this plan's tables (bdattn_plan_keep_tables), whose
  // calls then skip the upload; NULL when none.  Guarded by the library-wide
  // registry of kept workspaces, not by `mu`.
  const void *tables_at = nullptr;
};

namespace bdattn {
namespace abi {

// Records the thread-local error text and returns `code`.
int fail(int code, const std::string &msg);

// Argument checks of the forward entry points (before any HIP call): the clean
// segment as a table of buffers, or in one buffer.
int check_fwd_shards(const bdattn_plan *pl, const void *q, const bdattn_kv_shards *kv, const void *k1,
                     const void *v1, const void *o, int32_t o_dtype, const float *lse);
int check_fwd_args(const bdattn_plan *pl, const void *q, const void *k0, const void *v0, const void *k1,
                   const void *v1, const void *o, int32_t o_dtype, const float *lse);

// Launches the forward kernel reading the plan's tables at device address
// `tables` (laid out as the plan's image; only its forward prefix is read).
int launch_fwd_on_tables(const bdattn_plan *pl, const void *tables, const void *q, const void *k0, const void *v0,
                         const void *k1, const void *v1, void *o, int32_t o_dtype, float *lse, hipStream_t s);

int launch_fwd_shards(const bdattn_plan *pl, const void *tables, const void *q, const bdattn_kv_shards &kv,
                      const void *k1, const void *v1, void *o, int32_t o_dtype, float *lse, hipStream_t s);

// Bytes of the image prefix the forward kernel reads (header, row bounds, forward tiles).
int64_t fwd_table_bytes(const bdattn_plan *pl);

}  // namespace abi
}  // namespace bdattn
