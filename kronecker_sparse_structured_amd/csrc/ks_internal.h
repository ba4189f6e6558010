// ks_internal.h -- shared declarations between the libks host code and its
// HIP kernels. Not part of the public ABI (include/ks.h is).
#pragma once

#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

#include <hip/hip_runtime.h>

#include "ks.h"

namespace ks {

// Launches `kernel` and returns the status of this launch alone.
// hipLaunchKernel reports it directly; hipGetLastError would also return a
// failure left behind by an earlier, unrelated HIP call in this thread (for
// example a stream or event query that found work still pending).
template <typename... Params, size_t... I>
ks_status_t launch_kernel_impl(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                               hipStream_t stream, std::index_sequence<I...>, std::tuple<Params...>& p) {
    void* ptrs[] = {static_cast<void*>(&std::get<I>(p))..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream) == hipSuccess
               ? KS_OK
               : KS_ERR_HIP;
}

template <typename... Params, typename... Args>
ks_status_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                          Args&&... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    std::tuple<Params...> p(std::forward<Args>(args)...);
    return launch_kernel_impl(kernel, grid, block, lds, stream, std::index_sequence_for<Params...>{}, p);
}

// Element type codes for X and W.
enum ElemType : int { kF32 = 0, kBF16 = 1 };

inline int elem_bytes(int t) { return t == kBF16 ? 2 : 4; }

// Shape of one factor with its derived sizes (all below 2^31 after
// validation).
struct Shape {
    int a, b, c, d;
    int64_t n_in, n_out, nnz;
};

// Everything a launcher needs for one factor.
struct FactorCall {
    Shape s;
    int xt, wt;            // ElemType of X and W; Y is fp32
    const void* W;
    const void* X;
    float* Y;
    int64_t batch;
    hipStream_t stream;
    int num_cus;           // compute units of the current device
    int rows_per_block;    // 0 = default
    int store_waves;       // ks_store_waves_t (MFMA family)
};

// Kernel launchers. Each returns KS_OK, KS_ERR_UNSUPPORTED when the family
// cannot run this factor, or KS_ERR_HIP when the launch fails.
ks_status_t launch_generic(const FactorCall& f);
ks_status_t launch_valu(const FactorCall& f);
ks_status_t launch_mfma(const FactorCall& f);
ks_status_t launch_mfma_lds(const FactorCall& f);   // the same kernels

// Whether a family can run a factor (pure host; no HIP call).
bool valu_supports(const Shape& s, int xt, int wt);
bool mfma_supports(const Shape& s, int xt, int wt);
bool mfma_lds_supports(const Shape& s, int xt, int wt);

// Planner description of the VALU / MFMA tiles (pure host).
int valu_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len);
int mfma_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len);

// Fused pair of factors (intermediate kept in LDS). Returns KS_ERR_UNSUPPORTED
// when the pair does not fit the fused kernel.
bool fused_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1);
ks_status_t launch_fused_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1,
                              const void* W0, const void* W1, const void* X, float* Y,
                              int64_t batch, hipStream_t stream, int num_cus);

// Fused pair whose second factor works inside the first one's output slabs:
// F = (a, 16, 16, 16) then G = (16 a, 16, 16, 1). KS_ERR_UNSUPPORTED when the
// pair is not of that family.
bool slab_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1);
ks_status_t launch_slab_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1,
                             const void* W0, const void* W1, const void* X, float* Y,
                             int64_t batch, hipStream_t stream, int num_cus);

// A run of factors with whole rows resident in LDS (ks_rowchain.hip): n >= 2
// factors of small blocks whose widest row fits on chip. s, W: n entries.
bool row_chain_supports(const Shape* s, int n, int xt, int wt);
ks_status_t launch_row_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                             int64_t batch, hipStream_t stream);
int row_chain_describe(const Shape* s, int n, char* buf, size_t len);
// Gradients (ks_backward.hip). Blocks of W transposed into Wt (same element
// type); dK partial sums over row ranges in the workspace, then added in
// order (dw_workspace_bytes: 0 when one range covers the batch).
ks_status_t launch_transpose_blocks(const Shape& s, int wt, const void* W, void* Wt, hipStream_t stream);
size_t dw_workspace_bytes(const Shape& s, int xt, int64_t batch);
int dw_describe(const Shape& s, int xt, int64_t batch, char* buf, size_t len);
ks_status_t launch_dw(const Shape& s, int xt, const float* dY, const void* X, float* dK, int64_t batch, void* ws,
                      hipStream_t stream);

}  // namespace ks
