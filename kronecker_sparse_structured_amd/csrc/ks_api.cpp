// ks_api.cpp -- the C ABI of libks: argument validation, planning and
// dispatch. Validation is pure host code and returns before any HIP call, so
// every argument error can be produced without a GPU.
//
// The operation is Y = X * W^T for W with support I_a (x) 1_{b x c} (x) I_d
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph); see
// include/ks.h for the layouts.

#include <algorithm>
#include <array>
#include <map>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "ks_internal.h"

namespace {

using ks::Shape;

constexpr int64_t kLimit = int64_t(1) << 31;

ks_status_t shape_of(ks_pattern_t p, Shape* s) {
    if (p.a < 1 || p.b < 1 || p.c < 1 || p.d < 1) return KS_ERR_PATTERN;
    const int64_t a = p.a, b = p.b, c = p.c, d = p.d;
    const int64_t n_in = a * c * d, n_out = a * b * d;
    if (n_in >= kLimit || n_out >= kLimit) return KS_ERR_PATTERN;
    // a*b*c*d can overflow int64 only if the factors are huge; each partial
    // product is checked against 2^31 first.
    if (a * b >= kLimit || a * b * c >= kLimit || a * b * c * d >= kLimit) return KS_ERR_PATTERN;
    s->a = p.a; s->b = p.b; s->c = p.c; s->d = p.d;
    s->n_in = n_in; s->n_out = n_out; s->nnz = a * b * c * d;
    return KS_OK;
}

ks_status_t check_batch(int64_t batch) {
    return (batch < 0 || batch >= kLimit) ? KS_ERR_BATCH : KS_OK;
}

// The integer a C caller passed for an enum parameter. C allows any int
// there; in C++ loading a value outside the enum's range as the enum type is
// undefined, so the bits are read as an int instead.
template <typename E>
int enum_value(const E* e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, e, sizeof v);
    return v;
}

ks_status_t factor_types(int dt, int* xt, int* wt) {
    switch (dt) {
        case KS_DTYPE_F32: *xt = ks::kF32; *wt = ks::kF32; return KS_OK;
        case KS_DTYPE_BF16: *xt = ks::kBF16; *wt = ks::kBF16; return KS_OK;
        case KS_DTYPE_BF16W: *xt = ks::kF32; *wt = ks::kBF16; return KS_OK;
        default: return KS_ERR_DTYPE;
    }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [p, p+pb) and [q, q+qb) intersect.
bool overlap(const void* p, uint64_t pb, const void* q, uint64_t qb) {
    if (pb == 0 || qb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
    return a0 < b0 + qb && b0 < a0 + pb;
}

ks_status_t check_options(const ks_options_t* opt) {
    if (!opt) return KS_OK;
    if (opt->kernel < KS_KERNEL_AUTO || opt->kernel > KS_KERNEL_COLUMN) return KS_ERR_INVALID;
    if (opt->rows_per_block < 0 || opt->rows_per_block > 4096) return KS_ERR_INVALID;
    if (opt->store_waves < KS_STORE_AUTO || opt->store_waves > KS_STORE_DEDICATED) return KS_ERR_INVALID;
    if (opt->mfma_tile < 0 || opt->mfma_tile > KS_MFMA_TILES) return KS_ERR_INVALID;
    if (opt->mfma_loaders < 0 || opt->mfma_loaders > 2) return KS_ERR_INVALID;
    for (int i = 0; i < 3; ++i)
        if (opt->reserved[i] != 0) return KS_ERR_INVALID;
    return KS_OK;
}

// Compute units of the current device, cached per device id.
ks_status_t current_cus(int* cus) {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KS_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < static_cast<int>(cache.size()) && cache[dev] > 0) {
        *cus = cache[dev];
        return KS_OK;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return KS_ERR_HIP;
    if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
    cache[dev] = n;
    *cus = n;
    return KS_OK;
}

// The planner's table: for the patterns of a measured sweep, the fastest
// kernel family and store schedule (generated from the measurements by
// plan_table.py; the pages' "simple heuristic" on the pattern parameters has
// no published form, so it is fitted here).
struct PlanEntry {
    int a, b, c, d, xt, wt, kernel, store_waves, mfma_tile, mfma_loaders;
};
const PlanEntry kPlanTable[] = {
#include "ks_plan_table.inc"
    {0, 0, 0, 0, 0, 0, 0, 0, 0, 0}  // end
};

bool family_supports(int kernel, const Shape& s, int xt, int wt) {
    switch (kernel) {
        case KS_KERNEL_GENERIC: return true;
        case KS_KERNEL_VALU: return ks::valu_supports(s, xt, wt);
        case KS_KERNEL_MFMA: case KS_KERNEL_MFMA_LDS: return ks::mfma_supports(s, xt, wt);
        case KS_KERNEL_COLUMN: return ks::col_supports(s, xt, wt);
        default: return false;
    }
}

// The planner's kernel family (and, for the matrix-core family, store
// schedule) for one factor: the table's entry when the pattern and element
// types are in it; otherwise the column kernel for whole-slab tiles of 16 x
// 16 or 32 x 32 blocks, the matrix cores whenever the blocks fill 16 x 16
// tiles (measured faster than the VALU kernel from b = c = 16 up), else the
// VALU kernel, else the generic one.
struct Choice {
    int kernel, store_waves, mfma_tile, mfma_loaders;
};

Choice choose_kernel(const Shape& s, int xt, int wt) {
    for (const PlanEntry* e = kPlanTable; e->a != 0; ++e)
        if (e->a == s.a && e->b == s.b && e->c == s.c && e->d == s.d && e->xt == xt && e->wt == wt &&
            family_supports(e->kernel, s, xt, wt))
            return {e->kernel, e->store_waves, e->mfma_tile, e->mfma_loaders};
    if (ks::col_preferred(s, xt, wt)) return {KS_KERNEL_COLUMN, KS_STORE_AUTO, 0, 0};
    if (ks::mfma_supports(s, xt, wt)) return {KS_KERNEL_MFMA, KS_STORE_AUTO, 0, 0};
    if (ks::valu_supports(s, xt, wt)) return {KS_KERNEL_VALU, KS_STORE_AUTO, 0, 0};
    return {KS_KERNEL_GENERIC, KS_STORE_AUTO, 0, 0};
}

ks_status_t launch_family(int kernel, const ks::FactorCall& f) {
    switch (kernel) {
        case KS_KERNEL_GENERIC: return ks::launch_generic(f);
        case KS_KERNEL_VALU: return ks::launch_valu(f);
        case KS_KERNEL_MFMA: return ks::launch_mfma(f);
        case KS_KERNEL_MFMA_LDS: return ks::launch_mfma_lds(f);
        case KS_KERNEL_COLUMN: return ks::launch_col(f);
        default: return KS_ERR_INVALID;
    }
}

// A forced family runs or refuses; the planner's choice falls back to the
// generic kernel when its family refuses the call (for instance pointers
// that are not 16-byte aligned).
ks_status_t run_factor(int kernel, const ks::FactorCall& f) {
    if (kernel != KS_KERNEL_AUTO) return launch_family(kernel, f);
    const Choice chosen = choose_kernel(f.s, f.xt, f.wt);
    ks::FactorCall g = f;
    if (g.store_waves == KS_STORE_AUTO) g.store_waves = chosen.store_waves;
    if (g.mfma_tile == 0) g.mfma_tile = chosen.mfma_tile;
    if (g.mfma_loaders == 0) g.mfma_loaders = chosen.mfma_loaders;
    ks_status_t st = launch_family(chosen.kernel, g);
    if (st == KS_ERR_UNSUPPORTED &&
        (g.store_waves != f.store_waves || g.mfma_tile != f.mfma_tile || g.mfma_loaders != f.mfma_loaders))
        st = launch_family(chosen.kernel, f);
    if (st == KS_ERR_UNSUPPORTED && chosen.kernel != KS_KERNEL_GENERIC) st = ks::launch_generic(f);
    return st;
}

// Group kinds whose kernel needs 16-byte aligned input and output.
bool aligned_pair_kind(int kind) { return kind == 4 || kind == 5; }

// Validated chain: shapes, element types and the fusion grouping.
struct ChainPlan {
    std::vector<Shape> shapes;
    std::vector<int> group_start;  // first factor of each launch group
    std::vector<int> group_len;    // factors in the group (one launch)
    std::vector<int> group_kind;   // 0 single factor, 1 row-fused pair, 2 slab-fused pair,
                                   // 3 run of factors with rows resident in LDS,
                                   // 4 strided pair, 5 Monarch pair (both: 16-byte aligned
                                   // input and output only)
    int xt0 = ks::kF32, wt = ks::kF32;
    int64_t max_mid = 0;           // widest intermediate between groups
    int nbuf = 0;                  // workspace buffers (0, 1 or 2)
    size_t buf_bytes = 0;          // bytes per workspace buffer
};

// The closure rule (ks_closure.cpp) for a pair: whether a tile of its closed
// components with 16-byte X runs keeps its weights (at most 64 K values:
// half a compute unit's register file in fp32) and 16 rows of its
// intermediates (at most 128 KB of LDS) on chip, i.e. whether the pair can
// run as one pass that reads every X value once. Fused kernels may also
// split components and re-read X from L2 instead (the GPT-2 pair kernel does,
// for 8 beta0 a workgroup), so this reports rather than gates. Results are
// cached: the analysis is a union-find over the intermediate.
bool closure_fits(const Shape& f, const Shape& g) {
    static std::mutex mu;
    static std::map<std::array<int, 8>, bool> cache;
    const std::array<int, 8> key{f.a, f.b, f.c, f.d, g.a, g.b, g.c, g.d};
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    ks::Closure c;
    const bool fits = !ks::closure_of(f, g, &c) ||
                      (c.tile_weights <= 65536 && c.tile_components * c.mid * 16 * 4 <= 128 * 1024);
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() < 4096) cache.emplace(key, fits);
    return fits;
}

ks_status_t plan_chain(const ks_pattern_t* p, int n, int64_t batch, int dt,
                       unsigned flags, ChainPlan* plan) {
    if (!p) return KS_ERR_NULL;
    if (n < 1) return KS_ERR_CHAIN_MISMATCH;
    if (flags != KS_CHAIN_AUTO && flags != KS_CHAIN_NO_FUSE) return KS_ERR_INVALID;
    ks_status_t st = check_batch(batch);
    if (st != KS_OK) return st;
    st = factor_types(dt, &plan->xt0, &plan->wt);
    if (st != KS_OK) return st;
    plan->shapes.resize(n);
    for (int k = 0; k < n; ++k) {
        st = shape_of(p[k], &plan->shapes[k]);
        if (st != KS_OK) return st;
        if (k > 0 && plan->shapes[k - 1].n_out != plan->shapes[k].n_in) return KS_ERR_CHAIN_MISMATCH;
    }
    for (int k = 0; k < n;) {
        const int xt = (k == 0) ? plan->xt0 : ks::kF32;
        int len = 1, kind = 0;
        if (flags == KS_CHAIN_AUTO && k + 1 < n) {
            if (ks::fused_pair_supports(plan->shapes[k], plan->shapes[k + 1], xt, plan->wt, plan->wt)) {
                len = 2;
                kind = 1;
            } else if (ks::slab_pair_supports(plan->shapes[k], plan->shapes[k + 1], xt, plan->wt, plan->wt)) {
                len = 2;
                kind = 2;
            } else if (ks::strided_pair_supports(plan->shapes[k], plan->shapes[k + 1], xt, plan->wt, plan->wt)) {
                len = 2;
                kind = 4;
            } else if (ks::monarch_pair_supports(plan->shapes[k], plan->shapes[k + 1], xt, plan->wt, plan->wt)) {
                len = 2;
                kind = 5;
            } else {
                // the longest run from k whose rows (or closure tiles) fit on chip
                for (int m = n - k; m >= 2; --m) {
                    if (ks::row_chain_supports(&plan->shapes[k], m, xt, plan->wt)) {
                        len = m;
                        kind = 3;
                        break;
                    }
                }
                // but stop it earlier if that leaves the rest of the chain as one
                // whole radix-2/4 butterfly on each slab: the register-resident
                // kernel takes that (fp32 intermediates); the longest such rest
                // (measured: twelve factors on 4096-value slabs after two beat ten
                // on 1024-value slabs after four by 8 %)
                int slabs = 0;
                for (int m = 2; kind == 3 && m < len && k + len < n; ++m) {
                    if (n - k - m >= 2 &&
                        ks::resident_slab_form(&plan->shapes[k + m], n - k - m, ks::kF32, plan->wt, &slabs) &&
                        ks::row_chain_supports(&plan->shapes[k + m], n - k - m, ks::kF32, plan->wt)) {
                        len = m;
                        break;
                    }
                }
            }
        }
        plan->group_start.push_back(k);
        plan->group_len.push_back(len);
        plan->group_kind.push_back(kind);
        k += len;
    }
    const int groups = static_cast<int>(plan->group_start.size());
    for (int g = 0; g + 1 < groups; ++g) {
        const Shape& last = plan->shapes[plan->group_start[g] + plan->group_len[g] - 1];
        if (last.n_out > plan->max_mid) plan->max_mid = last.n_out;
    }
    plan->nbuf = groups <= 1 ? 0 : (groups == 2 ? 1 : 2);
    // A strided or Monarch pair that reads X or writes Y needs both 16-byte aligned;
    // otherwise it runs as its two factors, through a buffer that is neither
    // its input nor its output. The workspace does not depend on the
    // pointers, so it always has room for that.
    for (int g = 0; g < groups; ++g) {
        if (!aligned_pair_kind(plan->group_kind[g]) || (g != 0 && g != groups - 1)) continue;
        const Shape& first = plan->shapes[plan->group_start[g]];
        if (first.n_out > plan->max_mid) plan->max_mid = first.n_out;
        plan->nbuf = std::max(plan->nbuf, groups == 1 ? 1 : 2);
    }
    const uint64_t raw = static_cast<uint64_t>(batch) * static_cast<uint64_t>(plan->max_mid) * 4u;
    plan->buf_bytes = static_cast<size_t>((raw + 255u) / 256u * 256u);
    return KS_OK;
}

// ks_matmul and ks_matmul_ex with the dtype as the caller's int.
ks_status_t matmul_impl(ks_pattern_t p, const void* W, const void* X, void* Y, int64_t batch, int dt,
                        hipStream_t stream, const ks_options_t* opt) {
    ks_status_t st = check_options(opt);
    if (st != KS_OK) return st;
    Shape s;
    st = shape_of(p, &s);
    if (st != KS_OK) return st;
    st = check_batch(batch);
    if (st != KS_OK) return st;
    int xt = 0, wt = 0;
    st = factor_types(dt, &xt, &wt);
    if (st != KS_OK) return st;
    if (batch == 0) return KS_OK;
    if (!W || !X || !Y) return KS_ERR_NULL;
    if (!aligned(X, ks::elem_bytes(xt)) || !aligned(W, ks::elem_bytes(wt)) || !aligned(Y, 4))
        return KS_ERR_ALIGN;
    const uint64_t xb = static_cast<uint64_t>(batch) * s.n_in * ks::elem_bytes(xt);
    const uint64_t yb = static_cast<uint64_t>(batch) * s.n_out * 4u;
    const uint64_t wb = static_cast<uint64_t>(s.nnz) * ks::elem_bytes(wt);
    if (overlap(Y, yb, X, xb) || overlap(Y, yb, W, wb)) return KS_ERR_OVERLAP;

    const int kernel = opt ? opt->kernel : KS_KERNEL_AUTO;
    if (kernel == KS_KERNEL_VALU && !ks::valu_supports(s, xt, wt)) return KS_ERR_UNSUPPORTED;
    if (kernel == KS_KERNEL_MFMA && !ks::mfma_supports(s, xt, wt)) return KS_ERR_UNSUPPORTED;
    if (kernel == KS_KERNEL_MFMA_LDS && !ks::mfma_lds_supports(s, xt, wt)) return KS_ERR_UNSUPPORTED;
    if (kernel == KS_KERNEL_COLUMN && !ks::col_supports(s, xt, wt)) return KS_ERR_UNSUPPORTED;

    ks::FactorCall f;
    f.s = s; f.xt = xt; f.wt = wt; f.W = W; f.X = X; f.Y = static_cast<float*>(Y);
    f.batch = batch; f.stream = stream;
    f.rows_per_block = opt ? opt->rows_per_block : 0;
    f.store_waves = opt ? opt->store_waves : KS_STORE_AUTO;
    f.mfma_tile = opt ? opt->mfma_tile : 0;
    f.mfma_loaders = opt ? opt->mfma_loaders : 0;
    st = current_cus(&f.num_cus);
    if (st != KS_OK) return st;
    return run_factor(kernel, f);
}

// Arguments of ks_matmul_dw and ks_matmul_dw_noalloc other than the
// workspace: pattern, batch, dtype, pointers, alignment and overlaps of dW
// with the inputs. Returns the shape and X's element type.
ks_status_t dw_check(ks_pattern_t p, const void* dY, const void* X, const void* dW, int64_t batch, int dt, Shape* s,
                     int* xt) {
    ks_status_t st = shape_of(p, s);
    if (st != KS_OK) return st;
    st = check_batch(batch);
    if (st != KS_OK) return st;
    int wt = 0;
    st = factor_types(dt, xt, &wt);
    if (st != KS_OK) return st;
    if (!dW) return KS_ERR_NULL;
    if (batch > 0 && (!dY || !X)) return KS_ERR_NULL;
    if (!aligned(dW, 4) || (batch > 0 && (!aligned(dY, 4) || !aligned(X, ks::elem_bytes(*xt))))) return KS_ERR_ALIGN;
    const uint64_t gb = static_cast<uint64_t>(batch) * s->n_out * 4u;
    const uint64_t xb = static_cast<uint64_t>(batch) * s->n_in * ks::elem_bytes(*xt);
    const uint64_t wb = static_cast<uint64_t>(s->nnz) * 4u;
    if (overlap(dW, wb, dY, gb) || overlap(dW, wb, X, xb)) return KS_ERR_OVERLAP;
    return KS_OK;
}

}  // namespace

extern "C" {

const char* ks_status_string(ks_status_t status) {
    switch (enum_value(&status)) {
        case KS_OK: return "KS_OK";
        case KS_ERR_NULL: return "KS_ERR_NULL: a required pointer is NULL";
        case KS_ERR_PATTERN: return "KS_ERR_PATTERN: pattern field < 1 or size >= 2^31";
        case KS_ERR_BATCH: return "KS_ERR_BATCH: batch < 0 or >= 2^31";
        case KS_ERR_DTYPE: return "KS_ERR_DTYPE: unsupported dtype";
        case KS_ERR_CHAIN_MISMATCH: return "KS_ERR_CHAIN_MISMATCH: chain is empty or widths do not match";
        case KS_ERR_WORKSPACE: return "KS_ERR_WORKSPACE: workspace missing or too small";
        case KS_ERR_ALIGN: return "KS_ERR_ALIGN: pointer not aligned to its element size";
        case KS_ERR_OVERLAP: return "KS_ERR_OVERLAP: output or workspace overlaps an input";
        case KS_ERR_HIP: return "KS_ERR_HIP: a HIP call failed";
        case KS_ERR_UNSUPPORTED: return "KS_ERR_UNSUPPORTED: the forced kernel cannot run this pattern";
        case KS_ERR_INVALID: return "KS_ERR_INVALID: invalid flags or options";
    }
    return "KS_ERR_UNKNOWN";
}

const char* ks_version(void) { return "libks 0.1.0 gfx950"; }

ks_status_t ks_matmul_ex(ks_pattern_t p, const void* W, const void* X, void* Y,
                         int64_t batch, ks_dtype_t dt, hipStream_t stream,
                         const ks_options_t* opt) {
    return matmul_impl(p, W, X, Y, batch, enum_value(&dt), stream, opt);
}

ks_status_t ks_matmul(ks_pattern_t p, const void* W, const void* X, void* Y,
                      int64_t batch, ks_dtype_t dt, hipStream_t stream) {
    return matmul_impl(p, W, X, Y, batch, enum_value(&dt), stream, nullptr);
}

ks_status_t ks_matmul_dx_workspace_size(ks_pattern_t p, ks_dtype_t dt, size_t* bytes) {
    if (!bytes) return KS_ERR_NULL;
    Shape s;
    ks_status_t st = shape_of(p, &s);
    if (st != KS_OK) return st;
    int xt = 0, wt = 0;
    st = factor_types(enum_value(&dt), &xt, &wt);
    if (st != KS_OK) return st;
    *bytes = (static_cast<size_t>(s.nnz) * ks::elem_bytes(wt) + 255) / 256 * 256;
    return KS_OK;
}

ks_status_t ks_matmul_dx(ks_pattern_t p, const void* W, const void* dY, void* dX, int64_t batch,
                         ks_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream) {
    Shape s;
    ks_status_t st = shape_of(p, &s);
    if (st != KS_OK) return st;
    st = check_batch(batch);
    if (st != KS_OK) return st;
    int xt = 0, wt = 0;
    st = factor_types(enum_value(&dt), &xt, &wt);
    if (st != KS_OK) return st;
    if (batch == 0) return KS_OK;
    if (!W || !dY || !dX) return KS_ERR_NULL;
    size_t need = 0;
    ks_matmul_dx_workspace_size(p, dt, &need);
    if (!ws || ws_bytes < need) return KS_ERR_WORKSPACE;
    if (!aligned(dY, ks::elem_bytes(xt)) || !aligned(W, ks::elem_bytes(wt)) || !aligned(dX, 4) || !aligned(ws, 16))
        return KS_ERR_ALIGN;
    const uint64_t gb = static_cast<uint64_t>(batch) * s.n_out * ks::elem_bytes(xt);
    const uint64_t xb = static_cast<uint64_t>(batch) * s.n_in * 4u;
    const uint64_t wb = static_cast<uint64_t>(s.nnz) * ks::elem_bytes(wt);
    if (overlap(dX, xb, dY, gb) || overlap(dX, xb, W, wb) || overlap(dX, xb, ws, need) ||
        overlap(ws, need, dY, gb) || overlap(ws, need, W, wb))
        return KS_ERR_OVERLAP;
    // dX = dY W: the forward product of pattern (a, c, b, d) whose blocks are
    // W's blocks transposed
    st = ks::launch_transpose_blocks(s, wt, W, ws, stream);
    if (st != KS_OK) return st;
    Shape st_s;
    ks_pattern_t pt = {p.a, p.c, p.b, p.d};
    st = shape_of(pt, &st_s);
    if (st != KS_OK) return st;
    ks::FactorCall f;
    f.s = st_s; f.xt = xt; f.wt = wt; f.W = ws; f.X = dY; f.Y = static_cast<float*>(dX);
    f.batch = batch; f.stream = stream; f.rows_per_block = 0; f.store_waves = KS_STORE_AUTO;
    st = current_cus(&f.num_cus);
    if (st != KS_OK) return st;
    return run_factor(KS_KERNEL_AUTO, f);
}

ks_status_t ks_matmul_dw_workspace_size(ks_pattern_t p, int64_t batch, ks_dtype_t dt, size_t* bytes) {
    if (!bytes) return KS_ERR_NULL;
    Shape s;
    ks_status_t st = shape_of(p, &s);
    if (st != KS_OK) return st;
    st = check_batch(batch);
    if (st != KS_OK) return st;
    int xt = 0, wt = 0;
    st = factor_types(enum_value(&dt), &xt, &wt);
    if (st != KS_OK) return st;
    *bytes = ks::dw_workspace_bytes(s, xt, batch);
    return KS_OK;
}

ks_status_t ks_matmul_dw(ks_pattern_t p, const void* dY, const void* X, void* dW, int64_t batch,
                         ks_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream) {
    Shape s;
    int xt = 0;
    ks_status_t st = dw_check(p, dY, X, dW, batch, enum_value(&dt), &s, &xt);
    if (st != KS_OK) return st;
    const size_t need = ks::dw_workspace_bytes(s, xt, batch);
    if (need > 0 && (!ws || ws_bytes < need)) return KS_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 16)) return KS_ERR_ALIGN;
    const uint64_t gb = static_cast<uint64_t>(batch) * s.n_out * 4u;
    const uint64_t xb = static_cast<uint64_t>(batch) * s.n_in * ks::elem_bytes(xt);
    const uint64_t wb = static_cast<uint64_t>(s.nnz) * 4u;
    if (overlap(dW, wb, ws, need) || overlap(ws, need, dY, gb) || overlap(ws, need, X, xb)) return KS_ERR_OVERLAP;
    return ks::launch_dw(s, xt, static_cast<const float*>(dY), X, static_cast<float*>(dW), batch, ws, stream);
}

ks_status_t ks_matmul_dw_noalloc(ks_pattern_t p, const void* dY, const void* X, void* dW, int64_t batch,
                                 ks_dtype_t dt, hipStream_t stream) {
    Shape s;
    int xt = 0;
    ks_status_t st = dw_check(p, dY, X, dW, batch, enum_value(&dt), &s, &xt);
    if (st != KS_OK) return st;
    const size_t need = ks::dw_workspace_bytes(s, xt, batch);
    if (need > ks::dw_scratch_bytes()) return KS_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        // this device's copy of the library's scratch array
        st = ks::dw_scratch(&ws);
        if (st != KS_OK) return st;
    }
    return ks::launch_dw(s, xt, static_cast<const float*>(dY), X, static_cast<float*>(dW), batch, ws, stream);
}

ks_status_t ks_chain_workspace_size(const ks_pattern_t* p, int n, int64_t batch,
                                    ks_dtype_t dt, unsigned flags, size_t* bytes) {
    if (!bytes) return KS_ERR_NULL;
    ChainPlan plan;
    ks_status_t st = plan_chain(p, n, batch, enum_value(&dt), flags, &plan);
    if (st != KS_OK) return st;
    *bytes = (batch == 0) ? 0 : static_cast<size_t>(plan.nbuf) * plan.buf_bytes;
    return KS_OK;
}

ks_status_t ks_chain_plan(const ks_pattern_t* p, int n, int64_t batch, ks_dtype_t dt,
                          unsigned flags, int* group_len, int cap, int* groups) {
    if (!groups || (cap > 0 && !group_len)) return KS_ERR_NULL;
    ChainPlan plan;
    ks_status_t st = plan_chain(p, n, batch, enum_value(&dt), flags, &plan);
    if (st != KS_OK) return st;
    const int ng = static_cast<int>(plan.group_len.size());
    *groups = ng;
    for (int g = 0; g < ng && g < cap; ++g) group_len[g] = plan.group_len[g];
    return KS_OK;
}

ks_status_t ks_chain_matmul(const ks_pattern_t* p, int n, const void* const* W,
                            const void* X, void* Y, int64_t batch, ks_dtype_t dt,
                            void* ws, size_t ws_bytes, unsigned flags,
                            hipStream_t stream) {
    ChainPlan plan;
    ks_status_t st = plan_chain(p, n, batch, enum_value(&dt), flags, &plan);
    if (st != KS_OK) return st;
    if (batch == 0) return KS_OK;
    if (!W || !X || !Y) return KS_ERR_NULL;
    for (int k = 0; k < n; ++k)
        if (!W[k]) return KS_ERR_NULL;
    const size_t need = static_cast<size_t>(plan.nbuf) * plan.buf_bytes;
    if (need > 0 && (!ws || ws_bytes < need)) return KS_ERR_WORKSPACE;
    const int xe = ks::elem_bytes(plan.xt0), we = ks::elem_bytes(plan.wt);
    if (!aligned(X, xe) || !aligned(Y, 4)) return KS_ERR_ALIGN;
    for (int k = 0; k < n; ++k)
        if (!aligned(W[k], we)) return KS_ERR_ALIGN;
    if (need > 0 && !aligned(ws, 16)) return KS_ERR_ALIGN;
    const uint64_t xb = static_cast<uint64_t>(batch) * plan.shapes[0].n_in * xe;
    const uint64_t yb = static_cast<uint64_t>(batch) * plan.shapes[n - 1].n_out * 4u;
    if (overlap(Y, yb, X, xb)) return KS_ERR_OVERLAP;
    if (need > 0 && (overlap(ws, need, X, xb) || overlap(ws, need, Y, yb))) return KS_ERR_OVERLAP;
    for (int k = 0; k < n; ++k) {
        const uint64_t wb = static_cast<uint64_t>(plan.shapes[k].nnz) * we;
        if (overlap(Y, yb, W[k], wb)) return KS_ERR_OVERLAP;
        if (need > 0 && overlap(ws, need, W[k], wb)) return KS_ERR_OVERLAP;
    }

    int cus = 0;
    st = current_cus(&cus);
    if (st != KS_OK) return st;
    char* bufs[2] = {static_cast<char*>(ws), static_cast<char*>(ws) + plan.buf_bytes};
    const void* cur = X;
    int cur_t = plan.xt0;
    const int groups = static_cast<int>(plan.group_start.size());
    for (int g = 0; g < groups; ++g) {
        const int k = plan.group_start[g];
        float* out = (g == groups - 1) ? static_cast<float*>(Y)
                                       : reinterpret_cast<float*>(bufs[g % 2]);
        if (plan.group_kind[g] == 1) {
            st = ks::launch_fused_pair(plan.shapes[k], plan.shapes[k + 1], cur_t, plan.wt, plan.wt,
                                       W[k], W[k + 1], cur, out, batch, stream, cus);
        } else if (plan.group_kind[g] == 2) {
            st = ks::launch_slab_pair(plan.shapes[k], plan.shapes[k + 1], cur_t, plan.wt, plan.wt,
                                      W[k], W[k + 1], cur, out, batch, stream, cus);
        } else if (plan.group_kind[g] == 3) {
            st = ks::launch_row_chain(&plan.shapes[k], plan.group_len[g], cur_t, plan.wt, W + k, cur, out, batch,
                                      stream, cus);
        } else if (plan.group_kind[g] == 4 && ks::strided_pair_aligned(cur, out)) {
            st = ks::launch_strided_pair(plan.shapes[k], plan.shapes[k + 1], cur_t, plan.wt, plan.wt, W[k], W[k + 1],
                                         cur, out, batch, stream, cus);
        } else if (plan.group_kind[g] == 5 && ks::monarch_pair_aligned(cur, out)) {
            st = ks::launch_monarch_pair(plan.shapes[k], plan.shapes[k + 1], cur_t, plan.wt, plan.wt, W[k], W[k + 1],
                                         cur, out, batch, stream, cus);
        } else if (aligned_pair_kind(plan.group_kind[g])) {
            // X or Y not 16-byte aligned: the two factors one at a time,
            // through the buffer that is neither this group's input nor output
            float* mid = reinterpret_cast<float*>(
                (cur == bufs[0] || out == reinterpret_cast<float*>(bufs[0])) ? bufs[1] : bufs[0]);
            // only the first or last group can see an unaligned pointer, and
            // the plan keeps a spare buffer for it
            if (plan.nbuf == 0 || static_cast<const void*>(mid) == cur || mid == out) return KS_ERR_UNSUPPORTED;
            ks::FactorCall f;
            f.s = plan.shapes[k]; f.xt = cur_t; f.wt = plan.wt; f.W = W[k]; f.X = cur; f.Y = mid;
            f.batch = batch; f.stream = stream; f.num_cus = cus; f.rows_per_block = 0;
            f.store_waves = KS_STORE_AUTO;
            st = run_factor(KS_KERNEL_AUTO, f);
            if (st == KS_OK) {
                f.s = plan.shapes[k + 1]; f.xt = ks::kF32; f.W = W[k + 1]; f.X = mid; f.Y = out;
                st = run_factor(KS_KERNEL_AUTO, f);
            }
        } else {
            ks::FactorCall f;
            f.s = plan.shapes[k]; f.xt = cur_t; f.wt = plan.wt; f.W = W[k]; f.X = cur; f.Y = out;
            f.batch = batch; f.stream = stream; f.num_cus = cus; f.rows_per_block = 0;
            f.store_waves = KS_STORE_AUTO;
            st = run_factor(KS_KERNEL_AUTO, f);
        }
        if (st != KS_OK) return st;
        cur = out;
        cur_t = ks::kF32;
    }
    return KS_OK;
}

ks_status_t ks_plan_describe(ks_pattern_t p, int64_t batch, ks_dtype_t dt, char* buf, size_t len) {
    if (!buf || len == 0) return KS_ERR_NULL;
    Shape s;
    ks_status_t st = shape_of(p, &s);
    if (st != KS_OK) return st;
    st = check_batch(batch);
    if (st != KS_OK) return st;
    int xt = 0, wt = 0;
    st = factor_types(enum_value(&dt), &xt, &wt);
    if (st != KS_OK) return st;
    const Choice choice = choose_kernel(s, xt, wt);
    const int kernel = choice.kernel;
    const int cus = 256;  // description only; launches use the device's count
    if (kernel == KS_KERNEL_COLUMN) ks::col_describe(s, xt, wt, batch, cus, buf, len);
    else if (kernel == KS_KERNEL_VALU) ks::valu_describe(s, xt, wt, batch, cus, buf, len);
    else if (kernel == KS_KERNEL_MFMA)
        ks::mfma_describe(s, xt, wt, batch, cus, buf, len, choice.store_waves, choice.mfma_tile,
                          choice.mfma_loaders);
    else std::snprintf(buf, len, "generic: one thread per output");
    return KS_OK;
}

ks_status_t ks_pair_closure(ks_pattern_t f, ks_pattern_t g, ks_closure_t* out) {
    if (!out) return KS_ERR_NULL;
    Shape sf, sg;
    ks_status_t st = shape_of(f, &sf);
    if (st != KS_OK) return st;
    st = shape_of(g, &sg);
    if (st != KS_OK) return st;
    if (sf.n_out != sg.n_in) return KS_ERR_CHAIN_MISMATCH;
    ks::Closure c;
    if (!ks::closure_of(sf, sg, &c)) return KS_ERR_UNSUPPORTED;
    out->components = c.components;
    out->mid = c.mid;
    out->inputs = c.inputs;
    out->outputs = c.outputs;
    out->weights = c.weights;
    out->in_run = c.in_run;
    out->out_run = c.out_run;
    out->tile_components = c.tile_components;
    out->tile_weights = c.tile_weights;
    out->uniform = c.uniform ? 1 : 0;
    out->reserved = 0;
    return KS_OK;
}

ks_status_t ks_chain_describe(const ks_pattern_t* p, int n, int64_t batch, ks_dtype_t dt, unsigned flags, char* buf,
                              size_t len) {
    if (!buf || len == 0) return KS_ERR_NULL;
    ChainPlan plan;
    ks_status_t st = plan_chain(p, n, batch, enum_value(&dt), flags, &plan);
    if (st != KS_OK) return st;
    buf[0] = '\0';
    size_t used = 0;
    const int groups = static_cast<int>(plan.group_start.size());
    for (int g = 0; g < groups && used + 1 < len; ++g) {
        const int k = plan.group_start[g];
        const Shape& s0 = plan.shapes[k];
        const int xt = g == 0 ? plan.xt0 : ks::kF32;
        char part[512];
        part[0] = '\0';
        switch (plan.group_kind[g]) {
            case 1:
            case 2:
            case 4:
            case 5: {
                static const char* const names[] = {"", "fused pair (shared rows)", "slab pair", "", "strided pair",
                                                    "Monarch pair"};
                const Shape& s1 = plan.shapes[k + 1];
                std::snprintf(part, sizeof part, "%s (%d, %d, %d, %d) -> (%d, %d, %d, %d), one launch",
                              names[plan.group_kind[g]], s0.a, s0.b, s0.c, s0.d, s1.a, s1.b, s1.c, s1.d);
                break;
            }
            case 3:
                ks::row_chain_describe(&plan.shapes[k], plan.group_len[g], part, sizeof part);
                break;
            default: {
                const ks_pattern_t pk = p[k];
                const int fdt = xt == ks::kBF16 ? KS_DTYPE_BF16 : (plan.wt == ks::kBF16 ? KS_DTYPE_BF16W : KS_DTYPE_F32);
                ks_plan_describe(pk, batch, static_cast<ks_dtype_t>(fdt), part, sizeof part);
            }
        }
        // the closure of the pair that this group's boundary splits
        char note[224];
        note[0] = '\0';
        const int last = k + plan.group_len[g] - 1;
        ks::Closure cl;
        if (flags == KS_CHAIN_AUTO && g + 1 < groups && ks::closure_of(plan.shapes[last], plan.shapes[last + 1], &cl))
            std::snprintf(note, sizeof note,
                          " (pair %d-%d unfused: %lld closed components of %lld values, 16-byte-run tile of %lld: "
                          "%lld weights, %s)",
                          last, last + 1, static_cast<long long>(cl.components), static_cast<long long>(cl.mid),
                          static_cast<long long>(cl.tile_components), static_cast<long long>(cl.tile_weights),
                          closure_fits(plan.shapes[last], plan.shapes[last + 1])
                              ? "fits on chip, no fused kernel for this shape"
                              : "too large to fuse without re-reading X");
        const int w = std::snprintf(buf + used, len - used, "%s[%d..%d] %s%s", g ? "; " : "", k, last, part, note);
        if (w < 0) break;
        used = std::min(len - 1, used + static_cast<size_t>(w));
    }
    return KS_OK;
}

}  // extern "C"
