// ks_fused.hip -- fused pairs of KS factors (intermediate kept on chip).
// Not implemented yet: every pair runs as two launches.
#include "ks_internal.h"

namespace ks {

bool fused_pair_supports(const Shape&, const Shape&, int, int, int) { return false; }

ks_status_t launch_fused_pair(const Shape&, const Shape&, int, int, int, const void*, const void*,
                              const void*, float*, int64_t, hipStream_t, int) {
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
