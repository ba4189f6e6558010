// ks_backward.hip -- gradients of one KS factor, for a layer's backward pass.
//
// For Y = X * W^T with W's support I_a (x) 1_{b x c} (x) I_d (KS abstract
// page, taxoreview.com "dblp:303/4794", first paragraph) and dY = dL/dY:
//   dX = dY * W. W^T is again a KS matrix, of pattern (a, c, b, d) with every
//        b x c block transposed, so dX is the forward product of that
//        pattern; this file only transposes the blocks (nnz elements, into
//        the caller's workspace) and the forward kernels do the rest.
//   dK[alpha][delta][beta][gamma] = sum_n dY[n][alpha][beta][delta]
//                                         * X[n][alpha][gamma][delta]
//        (each K entry sits in W once). The generic kernel here gives every
//        thread one K entry and one range of rows; per-range partial sums go
//        to the workspace and a second kernel adds them in range order, so
//        the result does not depend on scheduling.

#include <algorithm>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

constexpr int kThreads = 256;

// Wt[blk][gamma][beta] = W[blk][beta][gamma] for blk < a*d.
template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_blocks_kernel(const T* __restrict__ W, T* __restrict__ Wt, int b,
                                                                    int c, int64_t nnz) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;   // index into Wt
    if (e >= nnz) return;
    const int64_t bc = int64_t(b) * c;
    const int64_t blk = e / bc;
    const int r = static_cast<int>(e - blk * bc);
    const int gamma = r / b, beta = r - gamma * b;
    Wt[e] = W[blk * bc + int64_t(beta) * c + gamma];
}

// One K entry per thread (gamma fastest, as K is stored), rows
// [split * rows_per_split, ...) of the batch; writes its partial sum to
// out[split * nnz + entry] (out is dK itself when there is one split).
template <typename TX>
__global__ __launch_bounds__(kThreads) void dw_generic_kernel(const float* __restrict__ dY, const TX* __restrict__ X,
                                                              float* __restrict__ out, int a, int b, int c, int d,
                                                              int64_t batch, int64_t rows_per_split, int64_t nnz) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= nnz) return;
    const int gamma = static_cast<int>(e % c);
    int64_t q = e / c;
    const int beta = static_cast<int>(q % b);
    q /= b;
    const int delta = static_cast<int>(q % d);
    const int alpha = static_cast<int>(q / d);
    const int64_t n_in = int64_t(a) * c * d, n_out = int64_t(a) * b * d;
    const int64_t n0 = int64_t(blockIdx.y) * rows_per_split;
    const int64_t n1 = min(batch, n0 + rows_per_split);
    const float* gy = dY + (int64_t(alpha) * b + beta) * d + delta;
    const TX* gx = X + (int64_t(alpha) * c + gamma) * d + delta;
    float acc = 0.0f;
    for (int64_t n = n0; n < n1; ++n) acc = fmaf(gy[n * n_out], to_f32(gx[n * n_in]), acc);
    out[int64_t(blockIdx.y) * nnz + e] = acc;
}

// dK[e] = sum over splits s (ascending) of part[s * nnz + e].
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(const float* __restrict__ part, float* __restrict__ dK,
                                                             int nsplit, int64_t nnz) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= nnz) return;
    float acc = 0.0f;
    for (int s = 0; s < nsplit; ++s) acc += part[int64_t(s) * nnz + e];
    dK[e] = acc;
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (e < n) p[e] = 0.0f;
}

unsigned grid_for(int64_t n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }

}  // namespace

ks_status_t launch_transpose_blocks(const Shape& s, int wt, const void* W, void* Wt, hipStream_t stream) {
    if (grid_for(s.nnz) == 0) return KS_OK;
    if (wt == kF32)
        return launch_kernel(transpose_blocks_kernel<float>, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream,
                             static_cast<const float*>(W), static_cast<float*>(Wt), s.b, s.c, s.nnz);
    return launch_kernel(transpose_blocks_kernel<bf16_t>, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream,
                         static_cast<const bf16_t*>(W), static_cast<bf16_t*>(Wt), s.b, s.c, s.nnz);
}

int dw_splits(const Shape& s, int64_t batch) {
    if (batch <= 1) return 1;
    // about 2048 workgroups, at most 256 ranges of rows, and partial sums
    // within 64 MB of workspace
    const int64_t groups = (s.nnz + kThreads - 1) / kThreads;
    int64_t splits = std::max<int64_t>(1, (2048 + groups - 1) / groups);
    splits = std::min<int64_t>(splits, std::min<int64_t>(batch, 256));
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, (int64_t(64) << 20) / (s.nnz * 4)));
    return static_cast<int>(splits);
}

size_t dw_workspace_bytes(const Shape& s, int64_t batch) {
    const int splits = dw_splits(s, batch);
    return splits <= 1 ? 0 : (static_cast<size_t>(splits) * s.nnz * 4 + 255) / 256 * 256;
}

ks_status_t launch_dw(const Shape& s, int xt, const float* dY, const void* X, float* dK, int64_t batch, void* ws,
                      hipStream_t stream) {
    if (batch == 0)
        return launch_kernel(fill_zero_kernel, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream, dK, s.nnz);
    const int splits = dw_splits(s, batch);
    const int64_t rps = (batch + splits - 1) / splits;
    float* out = splits > 1 ? static_cast<float*>(ws) : dK;
    const dim3 grid(grid_for(s.nnz), static_cast<unsigned>(splits));
    ks_status_t st;
    if (xt == kF32)
        st = launch_kernel(dw_generic_kernel<float>, grid, dim3(kThreads), 0, stream, dY, static_cast<const float*>(X),
                           out, s.a, s.b, s.c, s.d, batch, rps, s.nnz);
    else
        st = launch_kernel(dw_generic_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, dY,
                           static_cast<const bf16_t*>(X), out, s.a, s.b, s.c, s.d, batch, rps, s.nnz);
    if (st != KS_OK || splits == 1) return st;
    return launch_kernel(dw_reduce_kernel, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(ws), dK, splits, s.nnz);
}

}  // namespace ks
