// ks_digitchain.hip -- a run of square power-of-two KS factors in one launch,
// several factors per LDS round trip.
//
// Chains of KS factors are the Butterfly (and Monarch) layers (KS abstract
// page, taxoreview.com "dblp:303/4794", first paragraph, first sentence); a
// radix-2 or radix-4 butterfly is a run of factors (a, b, b, d) with every
// size a power of two. Write a row index in binary. Factor (a, b, b, d)
// reads the row as X[alpha][gamma][delta] (delta the low log2 d bits, gamma
// the next log2 b bits, alpha the rest) and writes Y[alpha][beta][delta]: it
// mixes only the bits [log2 d, log2 d + log2 b) of the index (its "digit"),
// with a b x b block K[alpha][delta] chosen by the other bits.
//
// A thread that holds the S values of a row whose indices differ only in the
// digits of M consecutive factors (S = b^M <= 16) can apply all M factors in
// registers, if it also holds their blocks for its column (the fixed other
// bits): M * S * b weights, at most 128 registers. The run is cut into such
// passes; between passes the row goes through LDS once. A radix-2 chain on
// n = 1024 (ten factors) takes three round trips instead of ten.
//
// Digits of a pass are ordered by address (ascending or descending along
// the chain: both butterfly orders), so that the e-th held value sits at
// index base(column) + sum_i digit_i(e) * place_i with digit i of e at
// compile-time position i. Threads take consecutive columns (the index bits
// outside the pass's digits, low bits first) and, while a column's weights
// are in registers, as many rows as the workgroup holds.
//
// LDS layout: row r, index i at r * n + swz(i), swz(i) = i ^ (4 * (i / 64)
// mod 64): index bits 6..9 are folded into bits 2..5, which spreads the 64
// lanes of every pass of a butterfly over the banks while keeping runs of
// four (for 16-byte X loads and Y stores) together.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPasses = 12;           // factors (and passes) per launch: a 4096-wide radix-2 chain
constexpr int kMaxWidth = 4096;
// Two configurations, chosen per run (measured on 16,384 rows): at most 8
// values a thread (90 VGPRs, five waves a SIMD) with 32 KB of rows per
// workgroup, or at most 16 (204 VGPRs, two waves) with 64 KB. The first is
// faster on radix-2 chains and on widths up to 2048 (radix-2 n = 1024: 41 vs
// 46 us; radix-4 n = 1024: 44 vs 50 us); radix-4 chains on 4096-wide rows
// need the 16-value passes (two factors per pass) and the larger row block
// (277 vs 301 us).
struct Config {
    int smax, lds_bytes;
};
constexpr Config kSmall{8, 32 * 1024}, kLarge{16, 64 * 1024};

typedef float floatx4 __attribute__((ext_vector_type(4)));

struct PassDesc {
    int b, m, desc;          // radix, factors, 1: digits in descending address order along the chain
    int first;               // first factor of the pass (index into the run)
    int setmask;             // index bits the pass's digits cover
};

struct DigitArgs {
    int n, nbits;            // row width (power of two) and its log2
    int rows;                // rows per workgroup
    int npass;
    int64_t batch;
    int vec_x, vec_y;
    // arrays indexed at run time by pass or factor (see pick()), packed so
    // that the values a pick reads fit in scalar registers:
    // pass: b == 4 | m << 1 | desc << 4 | first << 5 | setmask << 9
    int pass[kMaxPasses];
    int fshift[kMaxPasses];  // factor: log2 d | log2(b d) << 8 (index >> log2(b d) = alpha)
    const void* w[kMaxPasses];
};

// The kernel reads its argument block through the kernel-argument segment
// pointer, in the constant address space: the arrays above are indexed by
// pass and factor at run time, which on a by-value copy would force the
// whole block into scratch memory; here each read is one scalar load. The
// block is the kernel's first argument, at offset 0 of the segment.
typedef const __attribute__((address_space(4))) DigitArgs KArgs;

__device__ __forceinline__ int swz(int i) { return i ^ ((i >> 4) & 60); }

__device__ __forceinline__ PassDesc pass_of(KArgs* args, int p) {
    const int v = args->pass[p];
    return PassDesc{(v & 1) ? 4 : 2, (v >> 1) & 7, (v >> 4) & 1, (v >> 5) & 15, v >> 9};
}
__device__ __forceinline__ int place_of(KArgs* args, int k) { return 1 << (args->fshift[k] & 255); }
__device__ __forceinline__ int ashift_of(KArgs* args, int k) { return args->fshift[k] >> 8; }

// index with the bits of c deposited, low first, into the bits of free
__device__ __forceinline__ int deposit(int c, int free, int nbits) {
    int out = 0;
    for (int bit = 0; bit < nbits; ++bit) {
        if ((free >> bit) & 1) {
            out |= (c & 1) << bit;
            c >>= 1;
        }
    }
    return out;
}

template <int B, int M>
struct PassShape {
    static constexpr int S = M == 1 ? B : M == 2 ? B * B : M == 3 ? B * B * B : B * B * B * B;
    static constexpr int U = S / B;          // blocks per factor in a column
};

__host__ __device__ constexpr int ipow(int b, int e) { return e == 0 ? 1 : b * ipow(b, e - 1); }

// Digit i (ascending address order) of a pass is factor j = i (ascending
// chains) or M - 1 - i (descending) of the pass.
template <int M, int DESC>
__device__ __forceinline__ int factor_of_digit(int i) { return DESC ? M - 1 - i : i; }

// First column of this thread in a pass with `cols` columns (every thread
// has one: cols and the block size are powers of two).
__device__ __forceinline__ int first_column(int cols) {
    return cols >= kThreads ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) % cols;
}

// The pass's weights for the column whose index bits outside the pass's
// digits are `base`, into wb: for factor j of the pass and the values u of
// its other digits, the block K_j[alpha][delta] (alpha = index >> log2(B d),
// delta = index mod d) at wb[((j U + u) B + beta) B + gamma].
template <int B, int M, int DESC, typename TW>
__device__ __forceinline__ void load_weights(float* wb, KArgs* args, const PassDesc& pd, int base) {
    using P = PassShape<B, M>;
    constexpr int U = P::U;
    int dplace[M];
#pragma unroll
    for (int i = 0; i < M; ++i) dplace[i] = place_of(args, pd.first + factor_of_digit<M, DESC>(i));
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const int i = DESC ? M - 1 - j : j;
        const int d = place_of(args, pd.first + j);
        const int ash = ashift_of(args, pd.first + j);
        const TW* K = static_cast<const TW*>(args->w[pd.first + j]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // e with digit i = 0 and the other digits from u
            const int e = (u % ipow(B, i)) + (u / ipow(B, i)) * ipow(B, i + 1);
            int off = 0;
#pragma unroll
            for (int q = 0; q < M; ++q) off += ((e / ipow(B, q)) % B) * dplace[q];
            const int idx = base + off;
            const TW* kp = K + (int64_t(idx >> ash) * d + (idx & (d - 1))) * (B * B);
#pragma unroll
            for (int k = 0; k < B * B; ++k) wb[(j * U + u) * B * B + k] = to_f32(kp[k]);
        }
    }
}

// One pass: factors first .. first + M - 1 of radix B, rows [0, nr) of the
// workgroup's LDS buffer, in place.
template <int B, int M, int DESC, typename TW>
__device__ __forceinline__ void run_pass(float* z, KArgs* args, const PassDesc& pd, int nr) {
    using P = PassShape<B, M>;
    constexpr int S = P::S, U = P::U;
    const int n = args->n;
    const int t = threadIdx.x;
    const int free = ((1 << args->nbits) - 1) & ~pd.setmask;
    const int cols = n / S;
    int dplace[M];
#pragma unroll
    for (int i = 0; i < M; ++i) dplace[i] = place_of(args, pd.first + factor_of_digit<M, DESC>(i));
    const int tpc = cols >= kThreads ? 1 : kThreads / cols;      // threads per column
    const int r0 = cols >= kThreads ? 0 : t / cols;
    for (int c = first_column(cols); c < cols; c += kThreads) {
        const int base = deposit(c, free, args->nbits);
        float wb[M * U * B * B];
        load_weights<B, M, DESC, TW>(wb, args, pd, base);
        int addr[S];                                             // swizzled LDS index of each held value
#pragma unroll
        for (int e = 0; e < S; ++e) {
            int off = 0;
#pragma unroll
            for (int i = 0; i < M; ++i) off += ((e / ipow(B, i)) % B) * dplace[i];
            addr[e] = swz(base + off);
        }
        for (int r = r0; r < nr; r += tpc) {
            float* zr = z + r * n;
            float v[S];
#pragma unroll
            for (int e = 0; e < S; ++e) v[e] = zr[addr[e]];
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const int i = DESC ? M - 1 - j : j;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e0 = (u % ipow(B, i)) + (u / ipow(B, i)) * ipow(B, i + 1);
                    const float* w = wb + (j * U + u) * B * B;
                    float x[B];
#pragma unroll
                    for (int ga = 0; ga < B; ++ga) x[ga] = v[e0 + ga * ipow(B, i)];
#pragma unroll
                    for (int be = 0; be < B; ++be) {
                        float acc = 0.0f;
#pragma unroll
                        for (int ga = 0; ga < B; ++ga) acc = fmaf(w[be * B + ga], x[ga], acc);
                        v[e0 + be * ipow(B, i)] = acc;
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < S; ++e) zr[addr[e]] = v[e];
        }
    }
}

// Dispatch on the pass's radix, length and direction; SMAX bounds the values
// a thread holds (and with them the weight registers: S * M * B).
template <typename TW, int SMAX>
__device__ __forceinline__ void pass_op(float* z, KArgs* args, const PassDesc& pd, int nr) {
#define KS_DIGIT_PASS(B_, M_, D_)                                                  \
    if (ipow(B_, M_) <= SMAX && pd.b == B_ && pd.m == M_ && pd.desc == D_) {       \
        run_pass<B_, M_, D_, TW>(z, args, pd, nr);                                 \
        return;                                                                    \
    }
    KS_DIGIT_PASS(2, 1, 0) KS_DIGIT_PASS(2, 2, 0) KS_DIGIT_PASS(2, 2, 1) KS_DIGIT_PASS(2, 3, 0)
    KS_DIGIT_PASS(2, 3, 1) KS_DIGIT_PASS(2, 4, 0) KS_DIGIT_PASS(2, 4, 1) KS_DIGIT_PASS(4, 1, 0)
    KS_DIGIT_PASS(4, 2, 0) KS_DIGIT_PASS(4, 2, 1)
#undef KS_DIGIT_PASS
}

template <typename TX, typename TW, int SMAX>
__global__ __launch_bounds__(kThreads) void digit_chain_kernel(DigitArgs block, const TX* __restrict__ X,
                                                               float* __restrict__ Y) {
    (void)block;                                 // read through the segment pointer
    KArgs* args = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    extern __shared__ __align__(16) float z[];
    const int n = args->n;
    const int64_t n0 = int64_t(blockIdx.x) * args->rows;
    const int nr = static_cast<int>(min(int64_t(args->rows), args->batch - n0));
    const int t = threadIdx.x;

    // X rows into LDS (bf16 widened exactly), runs of four kept together
    const TX* xs = X + n0 * n;
    if (args->vec_x) {
        const int q = n / 4;
        for (int k = t; k < nr * q; k += kThreads) {
            const int r = k / q, j = k - r * q;
            float v[4];
            load4_f32(xs + int64_t(r) * n + 4 * j, v);
            *reinterpret_cast<floatx4*>(z + r * n + swz(4 * j)) = floatx4{v[0], v[1], v[2], v[3]};
        }
    } else {
        for (int k = t; k < nr * n; k += kThreads) {
            const int r = k / n, j = k - r * n;
            z[r * n + swz(j)] = to_f32(xs[int64_t(r) * n + j]);
        }
    }
    __syncthreads();

    for (int p = 0; p < args->npass; ++p) {
        pass_op<TW, SMAX>(z, args, pass_of(args, p), nr);
        __syncthreads();
    }

    float* ys = Y + n0 * n;
    if (args->vec_y) {
        const int q = n / 4;
        for (int k = t; k < nr * q; k += kThreads) {
            const int r = k / q, j = k - r * q;
            const floatx4 v = *reinterpret_cast<const floatx4*>(z + r * n + swz(4 * j));
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(ys + int64_t(r) * n + 4 * j));
        }
    } else {
        for (int k = t; k < nr * n; k += kThreads) {
            const int r = k / n, j = k - r * n;
            ys[int64_t(r) * n + j] = z[r * n + swz(j)];
        }
    }
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int64_t v) {
    int l = 0;
    while ((int64_t(1) << l) < v) ++l;
    return l;
}

// Cut the run into passes: consecutive factors of one radix whose digits
// move monotonically along the index without overlapping, at most 16 values
// a thread. Returns the number of passes, or 0 if the run is not of this
// family.
int plan_passes(const Shape* s, int n, int smax, PassDesc* out) {
    if (n < 1 || n > kMaxPasses) return 0;
    const int64_t w = s[0].n_in;
    if (!pow2(w) || w > kMaxWidth || w < 2) return 0;
    for (int k = 0; k < n; ++k) {
        if (s[k].b != s[k].c || !(s[k].b == 2 || s[k].b == 4)) return 0;
        if (!pow2(s[k].a) || !pow2(s[k].d) || s[k].n_in != w || s[k].n_out != w) return 0;
    }
    int np = 0;
    for (int k = 0; k < n;) {
        const int b = s[k].b, q = log2i(b);
        const int mmax = log2i(smax) / q;
        PassDesc pd{b, 1, 0, k, ((b - 1) << log2i(s[k].d))};
        int last = log2i(s[k].d);
        int m = 1;
        while (m < mmax && k + m < n && s[k + m].b == b) {
            const int p = log2i(s[k + m].d);
            const int dir = p > last ? 0 : 1;
            if (m >= 2 && dir != pd.desc) break;
            if (dir == 0 && p < last + q) break;          // overlapping digits
            if (dir == 1 && p + q > last) break;
            pd.desc = dir;
            pd.setmask |= (b - 1) << p;
            last = p;
            ++m;
        }
        pd.m = m;
        if (np >= kMaxPasses) return 0;
        out[np++] = pd;
        k += m;
    }
    return np;
}

}  // namespace

template <int SMAX>
ks_status_t launch_typed(int xt, int wt, dim3 grid, size_t lds, hipStream_t stream, const DigitArgs& args,
                         const void* X, float* Y) {
    if (xt == kF32 && wt == kF32)
        return launch_kernel(digit_chain_kernel<float, float, SMAX>, grid, dim3(kThreads), lds, stream, args,
                             static_cast<const float*>(X), Y);
    if (xt == kBF16 && wt == kBF16)
        return launch_kernel(digit_chain_kernel<bf16_t, bf16_t, SMAX>, grid, dim3(kThreads), lds, stream, args,
                             static_cast<const bf16_t*>(X), Y);
    if (xt == kF32 && wt == kBF16)
        return launch_kernel(digit_chain_kernel<float, bf16_t, SMAX>, grid, dim3(kThreads), lds, stream, args,
                             static_cast<const float*>(X), Y);
    return KS_ERR_UNSUPPORTED;
}

Config config_for(const Shape* s, int n) {
    bool radix4 = true;
    for (int k = 0; k < n; ++k) radix4 = radix4 && s[k].b == 4;
    return (radix4 && s[0].n_in >= 4096) ? kLarge : kSmall;
}

bool digit_chain_supports(const Shape* s, int n, int xt, int wt) {
    (void)xt;
    (void)wt;
    PassDesc pd[kMaxPasses];
    return n >= 2 && n <= kMaxPasses && plan_passes(s, n, config_for(s, n).smax, pd) > 0;
}

ks_status_t launch_digit_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                               int64_t batch, hipStream_t stream) {
    DigitArgs args{};
    PassDesc pd[kMaxPasses];
    if (n < 2 || n > kMaxPasses) return KS_ERR_UNSUPPORTED;
    const Config cfg = config_for(s, n);
    args.npass = plan_passes(s, n, cfg.smax, pd);
    if (n < 2 || args.npass == 0) return KS_ERR_UNSUPPORTED;
    for (int p = 0; p < args.npass; ++p)
        args.pass[p] = (pd[p].b == 4 ? 1 : 0) | pd[p].m << 1 | pd[p].desc << 4 | pd[p].first << 5 | pd[p].setmask << 9;
    args.n = static_cast<int>(s[0].n_in);
    args.nbits = log2i(args.n);
    args.rows = std::max(1, std::min(1024, cfg.lds_bytes / (4 * args.n)));
    args.batch = batch;
    for (int k = 0; k < n; ++k) {
        args.fshift[k] = log2i(s[k].d) | log2i(int64_t(s[k].b) * s[k].d) << 8;
        args.w[k] = W[k];
    }
    const uintptr_t xa = reinterpret_cast<uintptr_t>(X), ya = reinterpret_cast<uintptr_t>(Y);
    args.vec_x = (args.n % 4 == 0 && xa % (xt == kBF16 ? 8 : 16) == 0) ? 1 : 0;
    args.vec_y = (args.n % 4 == 0 && ya % 16 == 0) ? 1 : 0;
    const int64_t blocks = (batch + args.rows - 1) / args.rows;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const size_t lds = size_t(args.rows) * args.n * 4;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (cfg.smax == 16) return launch_typed<16>(xt, wt, grid, lds, stream, args, X, Y);
    return launch_typed<8>(xt, wt, grid, lds, stream, args, X, Y);
}


int digit_chain_describe(const Shape* s, int n, char* buf, size_t len) {
    PassDesc pd[kMaxPasses];
    const Config cfg = config_for(s, n);
    const int np = plan_passes(s, n, cfg.smax, pd);
    const int w = static_cast<int>(s[0].n_in);
    int k = std::snprintf(buf, len, "digit-pass chain: %d factors in %d passes (", n, np);
    for (int p = 0; p < np && k > 0 && size_t(k) < len; ++p)
        k += std::snprintf(buf + k, len - k, "%s%dx radix %d", p ? ", " : "", pd[p].m, pd[p].b);
    if (k > 0 && size_t(k) < len)
        std::snprintf(buf + k, len - k, "), rows/wg=%d, lds=%d", std::max(1, std::min(1024, cfg.lds_bytes / (4 * w))),
                      std::max(1, std::min(1024, cfg.lds_bytes / (4 * w))) * w * 4);
    return 0;
}

}  // namespace ks
