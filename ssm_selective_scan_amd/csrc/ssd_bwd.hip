// ssd_bwd.hip — SSD backward with segment checkpoint-and-recompute.
#include "common.hpp"

namespace lr {

size_t ssd_bwd_workspace(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                         int64_t seg) {
  (void)B; (void)L; (void)H; (void)P; (void)G; (void)N; (void)seg;
  return 0;
}

hipError_t launch_ssd_bwd(int, const void*, const void*, const float*, const void*, const void*,
                          const float*, const float*, const void*, const float*, void*, void*,
                          float*, void*, void*, float*, float*, void*, int64_t, int64_t, int64_t,
                          int64_t, int64_t, int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace lr
