// ks_rowchain.hip -- a run of KS factors in one launch, whole rows resident
// in LDS.
//
// A chain of KS factors applied to a row (KS abstract page, taxoreview.com
// "dblp:303/4794", first paragraph: the Butterfly and Monarch layers are such
// chains) only ever mixes values of that row. When the widest row of the
// chain fits on chip, a workgroup can take R rows of X, apply every factor
// of the run in LDS (two row buffers, ping-pong) and write the R rows of Y:
// HBM sees X and Y once, whatever the number of factors, where one launch per
// factor moves every intermediate out and back. This is the case of deep
// chains of small blocks (b * c <= 16): radix-2 and radix-4 butterflies,
// Walsh-Hadamard products.
//
// Per factor (a, b, c, d), a thread owns (alpha, delta) groups: it loads the
// group's b x c weight block into registers once and, for each of its rows,
// reads the c inputs Z[r][alpha][gamma][delta] from LDS and writes the b
// outputs Z'[r][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
// * Z[r][alpha][gamma][delta] to the other buffer. Consecutive threads take
// consecutive delta, so LDS reads and writes of a wave are consecutive words
// when d >= 64 (strided by c or b words when d is small). A factor's
// weights (at most 64 KB here) are read once per workgroup, from the L2
// cache after the first. fp32 accumulation; intermediates are fp32 (bf16 X
// and weights are widened exactly).

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxFactors = 16;              // factors per launch
constexpr int kMaxWidth = 4096;              // widest row of the run (elements)
constexpr int kLdsTarget = 32 * 1024;        // LDS of the two row buffers (rows of 4096: 2 rows)
constexpr int64_t kMaxWeightBytes = 64 * 1024;
constexpr int kMaxBlock = 16;                // b * c held in registers

struct RowChainArgs {
    int nf;                  // factors in the run
    int pitch;               // LDS floats per row (widest row, multiple of 4)
    int rows;                // rows per workgroup
    int n_in, n_out;         // row widths of X and Y
    int64_t batch;
    int vec_x, vec_y;        // 1: rows of X / Y move as 4-element vectors
    int pat[kMaxFactors][4]; // (a, b, c, d) of each factor
    const void* w[kMaxFactors];
};

// Threads of one factor: with at least kThreads groups a thread takes
// groups t, t + kThreads, ... over all rows; with fewer, the rows of a group
// are dealt out to kThreads / groups threads.
struct ItemMap {
    int g0, gstep, r0, rstep;
};

__device__ __forceinline__ bool item_map(int groups, ItemMap* m) {
    const int t = threadIdx.x;
    if (groups >= kThreads) {
        *m = ItemMap{t, kThreads, 0, 1};
        return true;
    }
    const int tpg = kThreads / groups;
    *m = ItemMap{t % groups, groups, t / groups, tpg};
    return t / groups < tpg;
}

// One factor from src to dst (rows [0, nr) of the workgroup) with B x C
// blocks: a thread holds the B * C weights of its (alpha, delta) group in
// registers and applies them to each of its rows (C inputs read from LDS
// once, B outputs written).
template <int B, int C, typename TW>
__device__ __forceinline__ void apply_block(const float* src, float* dst, int pitch, int nr, int a, int d,
                                            const TW* __restrict__ K) {
    ItemMap m;
    if (!item_map(a * d, &m)) return;
    for (int g = m.g0; g < a * d; g += m.gstep) {
        const int alpha = g / d;
        const int delta = g - alpha * d;
        const TW* kp = K + int64_t(g) * (B * C);   // (alpha * d + delta) * b * c
        float w[B][C];
#pragma unroll
        for (int be = 0; be < B; ++be)
#pragma unroll
            for (int gm = 0; gm < C; ++gm) w[be][gm] = to_f32(kp[be * C + gm]);
        const float* s = src + alpha * C * d + delta;
        float* o = dst + alpha * B * d + delta;
        for (int r = m.r0; r < nr; r += m.rstep) {
            float x[C];
#pragma unroll
            for (int gm = 0; gm < C; ++gm) x[gm] = s[r * pitch + gm * d];
#pragma unroll
            for (int be = 0; be < B; ++be) {
                float acc = 0.0f;
#pragma unroll
                for (int gm = 0; gm < C; ++gm) acc = fmaf(w[be][gm], x[gm], acc);
                o[r * pitch + be * d] = acc;
            }
        }
    }
}

// Any b, c (up to 16): weights read from global memory (cached) per row.
template <typename TW>
__device__ __forceinline__ void apply_any(const float* src, float* dst, int pitch, int nr, int a, int b, int c,
                                          int d, const TW* __restrict__ K) {
    ItemMap m;
    if (!item_map(a * d, &m)) return;
    for (int g = m.g0; g < a * d; g += m.gstep) {
        const int alpha = g / d;
        const int delta = g - alpha * d;
        const TW* kp = K + int64_t(g) * b * c;
        const float* s = src + alpha * c * d + delta;
        float* o = dst + alpha * b * d + delta;
        for (int r = m.r0; r < nr; r += m.rstep) {
            for (int be = 0; be < b; ++be) {
                float acc = 0.0f;
                for (int gm = 0; gm < c; ++gm) acc = fmaf(to_f32(kp[be * c + gm]), s[r * pitch + gm * d], acc);
                o[r * pitch + be * d] = acc;
            }
        }
    }
}

// B x C blocks up to MAXBC weights take the register path (a kernel's VGPR
// count follows its largest block: MAXBC = 16 keeps it near 54 VGPRs, eight
// waves per SIMD).
template <int MAXBC, int B, int C, typename TW>
__device__ __forceinline__ bool try_block(const float* src, float* dst, int pitch, int nr, int a, int d,
                                          const TW* __restrict__ K) {
    if constexpr (B * C <= MAXBC) {
        apply_block<B, C>(src, dst, pitch, nr, a, d, K);
        return true;
    } else {
        return false;
    }
}

template <int MAXBC, int B, typename TW>
__device__ __forceinline__ void apply_b(const float* src, float* dst, int pitch, int nr, int a, int c, int d,
                                        const TW* __restrict__ K) {
    bool done = false;
    switch (c) {
        case 1: done = try_block<MAXBC, B, 1>(src, dst, pitch, nr, a, d, K); break;
        case 2: done = try_block<MAXBC, B, 2>(src, dst, pitch, nr, a, d, K); break;
        case 4: done = try_block<MAXBC, B, 4>(src, dst, pitch, nr, a, d, K); break;
        case 8: done = try_block<MAXBC, B, 8>(src, dst, pitch, nr, a, d, K); break;
        case 16: done = try_block<MAXBC, B, 16>(src, dst, pitch, nr, a, d, K); break;
    }
    if (!done) apply_any(src, dst, pitch, nr, a, B, c, d, K);
}

template <int MAXBC, typename TW>
__device__ __forceinline__ void apply_factor(const float* src, float* dst, int pitch, int nr, int a, int b, int c,
                                             int d, const TW* __restrict__ K) {
    switch (b) {
        case 1: apply_b<MAXBC, 1>(src, dst, pitch, nr, a, c, d, K); return;
        case 2: apply_b<MAXBC, 2>(src, dst, pitch, nr, a, c, d, K); return;
        case 4: apply_b<MAXBC, 4>(src, dst, pitch, nr, a, c, d, K); return;
        case 8: apply_b<MAXBC, 8>(src, dst, pitch, nr, a, c, d, K); return;
        case 16: apply_b<MAXBC, 16>(src, dst, pitch, nr, a, c, d, K); return;
    }
    apply_any(src, dst, pitch, nr, a, b, c, d, K);
}

template <typename TX, typename TW, int MAXBC>
__global__ __launch_bounds__(kThreads) void row_chain_kernel(const TX* __restrict__ X, float* __restrict__ Y,
                                                             RowChainArgs args) {
    extern __shared__ __align__(16) float zbuf[];
    const int pitch = args.pitch;
    // buffers as offsets from the LDS array itself (a pointer picked from an
    // array of pointers would lose its address space: generic accesses)
    const int bufsz = args.rows * pitch;
    const int64_t n0 = int64_t(blockIdx.x) * args.rows;
    const int nr = static_cast<int>(min(int64_t(args.rows), args.batch - n0));
    const int t = threadIdx.x;

    // X rows into buffer 0 (bf16 widened exactly)
    const TX* xs = X + n0 * args.n_in;
    if (args.vec_x) {
        const int q = args.n_in / 4;
        for (int i = t; i < nr * q; i += kThreads) {
            const int r = i / q, j = i - r * q;
            float v[4];
            load4_f32(xs + int64_t(r) * args.n_in + 4 * j, v);
            *reinterpret_cast<floatx4_t*>(zbuf + r * pitch + 4 * j) = floatx4_t{v[0], v[1], v[2], v[3]};
        }
    } else {
        for (int i = t; i < nr * args.n_in; i += kThreads) {
            const int r = i / args.n_in, j = i - r * args.n_in;
            zbuf[r * pitch + j] = to_f32(xs[int64_t(r) * args.n_in + j]);
        }
    }
    __syncthreads();

    for (int f = 0; f < args.nf; ++f) {
        const int a = args.pat[f][0], b = args.pat[f][1], c = args.pat[f][2], d = args.pat[f][3];
        const TW* K = static_cast<const TW*>(args.w[f]);
        const float* src = zbuf + (f & 1) * bufsz;
        float* dst = zbuf + ((f + 1) & 1) * bufsz;
        apply_factor<MAXBC>(src, dst, pitch, nr, a, b, c, d, K);
        __syncthreads();
    }

    // the last buffer to Y
    const float* z = zbuf + (args.nf & 1) * bufsz;
    float* ys = Y + n0 * args.n_out;
    if (args.vec_y) {
        const int q = args.n_out / 4;
        for (int i = t; i < nr * q; i += kThreads) {
            const int r = i / q, j = i - r * q;
            const floatx4_t v = *reinterpret_cast<const floatx4_t*>(z + r * pitch + 4 * j);
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4_t*>(ys + int64_t(r) * args.n_out + 4 * j));
        }
    } else {
        for (int i = t; i < nr * args.n_out; i += kThreads) {
            const int r = i / args.n_out, j = i - r * args.n_out;
            ys[int64_t(r) * args.n_out + j] = z[r * pitch + j];
        }
    }
}

// Rows per workgroup: two row buffers in kLdsTarget bytes (at least two rows,
// so that each weight block loaded serves more than one row).
int chain_rows(int pitch) {
    return std::max(2, std::min(16, kLdsTarget / (2 * 4 * pitch)));
}

int row_pitch(const Shape* s, int n) {
    int64_t w = s[0].n_in;
    for (int k = 0; k < n; ++k) w = std::max<int64_t>(w, s[k].n_out);
    return static_cast<int>((w + 3) / 4 * 4);
}

}  // namespace

bool row_chain_supports(const Shape* s, int n, int xt, int wt) {
    (void)xt;
    if (n < 2 || n > kMaxFactors) return false;
    int64_t w = s[0].n_in;
    for (int k = 0; k < n; ++k) {
        // small blocks only: with b * c = 64 the run measured no faster than one
        // launch per factor, with 128 2.4 times slower (VALU work and VGPRs)
        if (s[k].b * s[k].c > kMaxBlock) return false;
        if (s[k].nnz * elem_bytes(wt) > kMaxWeightBytes) return false;
        w = std::max<int64_t>(w, s[k].n_out);
    }
    return w <= kMaxWidth;
}

template <typename TX, typename TW>
ks_status_t launch_rc(int maxbc, dim3 grid, size_t lds, hipStream_t stream, const void* X, float* Y,
                      const RowChainArgs& args) {
    const TX* x = static_cast<const TX*>(X);
    if (maxbc > kMaxBlock) return KS_ERR_UNSUPPORTED;
    return launch_kernel(row_chain_kernel<TX, TW, kMaxBlock>, grid, dim3(kThreads), lds, stream, x, Y, args);
}

ks_status_t launch_row_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                             int64_t batch, hipStream_t stream, int num_cus) {
    if (!row_chain_supports(s, n, xt, wt)) return KS_ERR_UNSUPPORTED;
    if (resident_chain_supports(s, n, xt, wt) && resident_chain_aligned(X, Y))
        return launch_resident_chain(s, n, xt, wt, W, X, Y, batch, stream, num_cus);
    if (digit_chain_supports(s, n, xt, wt)) return launch_digit_chain(s, n, xt, wt, W, X, Y, batch, stream);
    RowChainArgs args{};
    args.nf = n;
    args.pitch = row_pitch(s, n);
    args.rows = chain_rows(args.pitch);
    args.n_in = static_cast<int>(s[0].n_in);
    args.n_out = static_cast<int>(s[n - 1].n_out);
    args.batch = batch;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(X), ya = reinterpret_cast<uintptr_t>(Y);
    const int xvec_align = xt == kBF16 ? 8 : 16;
    args.vec_x = (args.n_in % 4 == 0 && xa % xvec_align == 0) ? 1 : 0;
    args.vec_y = (args.n_out % 4 == 0 && ya % 16 == 0) ? 1 : 0;
    int maxbc = 1;
    for (int k = 0; k < n; ++k) {
        args.pat[k][0] = s[k].a;
        args.pat[k][1] = s[k].b;
        args.pat[k][2] = s[k].c;
        args.pat[k][3] = s[k].d;
        args.w[k] = W[k];
        maxbc = std::max(maxbc, s[k].b * s[k].c);
    }
    const int64_t blocks = (batch + args.rows - 1) / args.rows;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const size_t lds = size_t(2) * args.rows * args.pitch * 4;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (xt == kF32 && wt == kF32) return launch_rc<float, float>(maxbc, grid, lds, stream, X, Y, args);
    if (xt == kBF16 && wt == kBF16) return launch_rc<bf16_t, bf16_t>(maxbc, grid, lds, stream, X, Y, args);
    if (xt == kF32 && wt == kBF16) return launch_rc<float, bf16_t>(maxbc, grid, lds, stream, X, Y, args);
    return KS_ERR_UNSUPPORTED;
}

int row_chain_describe(const Shape* s, int n, char* buf, size_t len) {
    if (resident_chain_supports(s, n, kF32, kF32)) return resident_chain_describe(s, n, buf, len);
    if (digit_chain_supports(s, n, kF32, kF32)) return digit_chain_describe(s, n, buf, len);
    const int pitch = row_pitch(s, n);
    const int rows = chain_rows(pitch);
    return std::snprintf(buf, len, "row-resident chain: %d factors, rows/wg=%d, row pitch %d floats, lds=%d", n,
                         rows, pitch, 2 * rows * pitch * 4);
}

}  // namespace ks
