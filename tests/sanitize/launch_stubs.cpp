// Host-only stand-ins for the kernel launchers, for the sanitizer build of the
// scheduler and the C ABI.  The driver only takes paths that return before any
// launch, so reaching one of these is a bug in the validation: it aborts.
#include <cstdio>
#include <cstdlib>

#include "kernels/kernels.h"

namespace bdattn {

static hipError_t reached(const char *what) {
  std::fprintf(stderr, "launcher %s reached from the host-only build\n", what);
  std::abort();
}

hipError_t launch_fwd(const FwdArgs &, int32_t, hipStream_t) { return reached("fwd"); }
hipError_t launch_bwd(const BwdArgs &, int32_t, hipStream_t, bool, bool) { return reached("bwd"); }
hipError_t launch_prepare(const PrepArgs &, int32_t, hipStream_t) { return reached("prepare"); }
hipError_t launch_merge(int32_t, const void *, bool, const float *, int64_t, int32_t, int32_t, void *, bool, float *,
                        hipStream_t) {
  return reached("merge");
}
hipError_t launch_cast_bf16(const float *, void *, int64_t, hipStream_t) { return reached("cast"); }

}  // namespace bdattn
