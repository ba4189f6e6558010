// ks_mfma.hip -- placeholder until the matrix-core kernel lands.
#include <cstdio>

#include "ks_internal.h"

namespace ks {

bool mfma_supports(const Shape&, int, int) { return false; }

int mfma_describe(const Shape&, int, int, int64_t, int, char* buf, size_t len) {
    return std::snprintf(buf, len, "mfma: unsupported");
}

ks_status_t launch_mfma(const FactorCall&) { return KS_ERR_UNSUPPORTED; }

bool fused_pair_supports(const Shape&, const Shape&, int, int, int) { return false; }

ks_status_t launch_fused_pair(const Shape&, const Shape&, int, int, int, const void*, const void*,
                              const void*, float*, int64_t, hipStream_t, int) {
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
