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
    int mfma_tile = 0;     // 0 = planner choice, else a tile candidate 1..KS_MFMA_TILES (MFMA family)
    int mfma_loaders = 0;  // 0 = planner choice (one), 1 or 2 loader waves (MFMA family)
};

// Kernel launchers. Each returns KS_OK, KS_ERR_UNSUPPORTED when the family
// cannot run this factor, or KS_ERR_HIP when the launch fails.
ks_status_t launch_generic(const FactorCall& f);
ks_status_t launch_valu(const FactorCall& f);
ks_status_t launch_mfma(const FactorCall& f);
ks_status_t launch_mfma_lds(const FactorCall& f);   // the same kernels

// In-place column tiles for b = c in {16, 32} (ks_col.hip; fp32 X).
ks_status_t launch_col(const FactorCall& f);
bool col_supports(const Shape& s, int xt, int wt);
bool col_preferred(const Shape& s, int xt, int wt);   // the planner's choice
int col_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len);

// Whether a family can run a factor (pure host; no HIP call).
bool valu_supports(const Shape& s, int xt, int wt);
bool mfma_supports(const Shape& s, int xt, int wt);
bool mfma_lds_supports(const Shape& s, int xt, int wt);

// Planner description of the VALU / MFMA tiles (pure host).
int valu_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len);
int mfma_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len,
                  int store_waves = KS_STORE_AUTO, int mfma_tile = 0, int mfma_loaders = 0);

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

// Fused pair of butterfly-type factors F = (a, 16, 16, 16 e) then
// G = (16 a, 16, 16, e), e a multiple of 4 (ks_pair.hip): closed groups of 256
// values e apart. fp32 X only; X and Y must be 16-byte aligned
// (strided_pair_aligned), else the launcher returns KS_ERR_UNSUPPORTED.
bool strided_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1);
bool strided_pair_aligned(const void* X, const void* Y);
ks_status_t launch_strided_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                                const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                                int num_cus);

// Monarch-shaped pair F = (M, N, N, 1) then G = (1, M, M, N), M and N in
// {16, 32} (ks_monarch.hip): whole rows in LDS, weights streamed from L2.
// fp32 X (fp32 or bf16 weights) or bf16 X with bf16 weights; X and Y must be
// 16-byte aligned (monarch_pair_aligned), else the launcher returns
// KS_ERR_UNSUPPORTED.
bool monarch_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1);
bool monarch_pair_aligned(const void* X, const void* Y);
ks_status_t launch_monarch_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                                const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                                int num_cus);

// A run of factors with whole rows resident in LDS (ks_rowchain.hip): n >= 2
// factors of small blocks whose widest row fits on chip. s, W: n entries.
bool row_chain_supports(const Shape* s, int n, int xt, int wt);

// The same runs when every factor is square with b in {2, 4} and all sizes
// are powers of two (butterflies, Walsh-Hadamard): several factors per LDS
// round trip, in registers (ks_digitchain.hip). launch_row_chain takes it
// when it applies.
bool digit_chain_supports(const Shape* s, int n, int xt, int wt);
ks_status_t launch_digit_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                               int64_t batch, hipStream_t stream);
int digit_chain_describe(const Shape* s, int n, char* buf, size_t len);
// Whole radix-2 or radix-4 butterflies on 1024- or 4096-wide rows, every
// weight held in registers by one persistent workgroup a compute unit
// (ks_resident.hip); needs X and Y 16-byte aligned. launch_row_chain takes
// it first. The same on rows cut into slabs that each carry such a whole
// butterfly with their own blocks (every a divisible by the slab count):
// resident_slab_form finds the slab count, each workgroup keeps one slab's
// weights.
bool resident_chain_supports(const Shape* s, int n, int xt, int wt);
bool resident_slab_form(const Shape* s, int n, int xt, int wt, int* slabs);
bool resident_chain_aligned(const void* X, const float* Y);
ks_status_t launch_resident_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X,
                                  float* Y, int64_t batch, hipStream_t stream, int num_cus);
ks_status_t launch_resident_slabs(const Shape* s, int n, int slabs, int xt, int wt, const void* const* W,
                                  const void* X, float* Y, int64_t batch, hipStream_t stream, int num_cus);
int resident_chain_describe(const Shape* s, int n, int slabs, char* buf, size_t len);
// The closure rule for fusing factor f then g (ks_closure.cpp): closed
// components of the intermediate, with the largest component's sizes (in
// values) and the shortest runs of consecutive indices its X reads and Y
// writes form; a tile of components whose X reads come in 16-byte runs.
constexpr int64_t kMaxClosureMid = int64_t(1) << 22;
struct Closure {
    int64_t components;       // closed components
    int64_t mid;              // intermediates of the largest component
    int64_t inputs, outputs;  // its values of X read and of Y written
    int64_t weights;          // its weights (F blocks and G blocks)
    int64_t in_run, out_run;  // shortest runs of consecutive X and Y indices (component of index 0)
    int64_t tile_components;  // components per 16-byte-run tile
    int64_t tile_weights;     // weights of such a tile
    bool uniform;             // every component the same size
};
bool closure_of(const Shape& f, const Shape& g, Closure* c);
ks_status_t launch_row_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                             int64_t batch, hipStream_t stream, int num_cus);
int row_chain_describe(const Shape* s, int n, char* buf, size_t len);
// Gradients (ks_backward.hip). Blocks of W transposed into Wt (same element
// type); dK partial sums over row ranges in the workspace, then added in
// order (dw_workspace_bytes: 0 when one range covers the batch).
ks_status_t launch_transpose_blocks(const Shape& s, int wt, const void* W, void* Wt, hipStream_t stream);
size_t dw_workspace_bytes(const Shape& s, int xt, int64_t batch);
int dw_describe(const Shape& s, int xt, int64_t batch, char* buf, size_t len);
ks_status_t launch_dw(const Shape& s, int xt, const float* dY, const void* X, float* dK, int64_t batch, void* ws,
                      hipStream_t stream);
// The dK partial-sum scratch that ks_matmul_dw_noalloc uses instead of a
// caller's workspace: its size (every dw_workspace_bytes fits it), and this
// device's address of it (looked up once per device, on that device).
size_t dw_scratch_bytes();
ks_status_t dw_scratch(void** ptr);

}  // namespace ks
