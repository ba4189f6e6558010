// ks_generic.hip -- the fallback kernel: one thread per output element.
//
// Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
//                                    * X[n][alpha][gamma][delta]
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph: a
// support I_a (x) 1_{b x c} (x) I_d). Consecutive threads own consecutive
// outputs, so Y is written coalesced; X and K are read through the caches.
// Any pattern and any element types; used for small or irregular patterns
// and as a cross-check for the tiled kernels.

#include <algorithm>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void generic_kernel(const TX* __restrict__ X,
                                                      const TW* __restrict__ K,
                                                      float* __restrict__ Y, int a, int b,
                                                      int c, int d, int64_t total) {
    const int64_t n_out = int64_t(a) * b * d;
    const int64_t n_in = int64_t(a) * c * d;
    const int bd = b * d;
    const int64_t step = int64_t(gridDim.x) * blockDim.x;
    for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < total; idx += step) {
        const int64_t n = idx / n_out;
        const int j = static_cast<int>(idx - n * n_out);
        const int alpha = j / bd;
        const int rem = j - alpha * bd;
        const int beta = rem / d;
        const int delta = rem - beta * d;
        const TX* x = X + n * n_in + int64_t(alpha) * c * d + delta;
        const TW* k = K + ((int64_t(alpha) * d + delta) * b + beta) * c;
        float acc = 0.0f;
        for (int g = 0; g < c; ++g) acc = fmaf(to_f32(k[g]), to_f32(x[int64_t(g) * d]), acc);
        Y[idx] = acc;
    }
}

template <typename TX, typename TW>
ks_status_t launch_typed(const FactorCall& f) {
    const int64_t total = f.batch * f.s.n_out;
    const int64_t blocks_needed = (total + 255) / 256;
    const int64_t cap = int64_t(std::max(f.num_cus, 1)) * 64;
    const unsigned blocks = static_cast<unsigned>(std::max<int64_t>(1, std::min(blocks_needed, cap)));
    return launch_kernel(generic_kernel<TX, TW>, dim3(blocks), dim3(256), 0, f.stream,
                         static_cast<const TX*>(f.X), static_cast<const TW*>(f.W), f.Y,
                         f.s.a, f.s.b, f.s.c, f.s.d, total);
}

}  // namespace

ks_status_t launch_generic(const FactorCall& f) {
    if (f.xt == kF32 && f.wt == kF32) return launch_typed<float, float>(f);
    if (f.xt == kBF16 && f.wt == kBF16) return launch_typed<bf16_t, bf16_t>(f);
    if (f.xt == kF32 && f.wt == kBF16) return launch_typed<float, bf16_t>(f);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
