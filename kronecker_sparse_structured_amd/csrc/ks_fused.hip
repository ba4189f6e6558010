// ks_fused.hip -- two KS factors in one launch, the intermediate kept in LDS.
//
// Chains of KS factors are how Butterfly- and Monarch-type layers are built
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph). A pair
// F0 = (1, b0, c0, d0) followed by F1 = (a1, b1, c1, d1) with a1 = b0 and
// c1 * d1 = d0 has a simple joint structure: F1 reads F0's output row
// Z[beta0][delta0] as Z[alpha1][gamma1][delta1], i.e. alpha1 = beta0 and
// delta0 = gamma1 * d1 + delta1. Hence a fixed set of beta0 values (= alpha1
// values) needs all of X's row, produces a contiguous slab of Y's row
// (Y[alpha1][beta1][delta1]), and touches only its own slices of both weight
// tensors. The GPT-2-medium MLP shape (1, 64, 16, 64) -> (64, 8, 8, 8) is of
// this kind.
//
// Workgroup: 8 consecutive beta0 (= alpha1) values and a range of rows; one
// loader wave streams whole rows of X into an LDS ring (ks_stream.h); the 8
// workgroups that share rows run on the same XCD, so X is fetched from HBM
// once and served to the others from L2. Per stage of R rows, four consumer
// waves
//  (A) compute Z[r][beta0][delta0] for their 2 beta0 x 1 delta0 each
//      (c0 FMAs per value, weights in registers) into LDS,
//  (B) after an LDS barrier, compute Y[r][alpha1][beta1][delta1] for runs
//      of 4 delta1 (c1 FMAs per value, weights in registers) and store each
//      run as one 16-byte vector; a wave's stores cover 1 KB of a row.
// Z never leaves the chip: the pair moves |X| + |Y| + weights through HBM
// instead of |X| + 2|Z| + |Y|.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Shape family handled: F0 = (1, b0, 16, 64), F1 = (b0, 8, 8, 8), b0 % 8 == 0.
constexpr int kC0 = 16, kD0 = 64;          // first factor: gamma0, delta0 extents
constexpr int kB1 = 8, kC1 = 8, kD1 = 8;   // second factor: beta1, gamma1, delta1 extents
constexpr int kBT = 8;                     // beta0 (= alpha1) values per workgroup
constexpr int kRows = 4;                   // rows per stage
constexpr int kStages = 4;                 // LDS ring depth
constexpr int kInsts = kRows * kC0 * kD0 * 4 / 1024;   // loader instructions per fp32 stage
constexpr int kZPitch = kD0 + 8;           // Z row pitch per beta0 (floats), spreads LDS banks
static_assert(kRows % 2 == 0 && (kZPitch * 4) % 16 == 0, "phase B takes rows in pairs, Z in 16-byte runs");

struct FusedArgs {
    int b0;                 // beta0 extent (= alpha1 extent)
    int64_t n_in, n_mid, n_out;
    int64_t batch;
    int n_tiles;            // b0 / kBT
    int rows_per_split;     // multiple of kRows
};

template <typename TX, typename TW>
__global__ __launch_bounds__(kStreamThreads) void fused_pair_kernel(const TX* __restrict__ X,
                                                                    const TW* __restrict__ K0,
                                                                    const TW* __restrict__ K1,
                                                                    float* __restrict__ Y, FusedArgs args) {
    constexpr int EB = int(sizeof(TX));
    constexpr int VW = 16 / EB;
    constexpr int INSTS = kInsts * EB / 4;                 // a stage holds kRows whole rows of X
    constexpr int kStageBytes = INSTS * 1024;
    extern __shared__ __align__(16) unsigned char lds[];
    float* const zs = reinterpret_cast<float*>(lds + kStages * kStageBytes);   // [kRows][kBT][kZPitch]

    const int t = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    const int beta0 = tile * kBT;                          // first beta0 (= alpha1) of the tile

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kRows - 1) / kRows);

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        StageMap m;
        m.rows = kRows;
        m.blocks = 1;
        m.blk_vec = kC0 * kD0 / VW;                        // one whole row of X
        m.pad_vec = 0;
        m.row_vec = m.blk_vec;
        m.gstride = 0;
        LoaderPlan<INSTS> lp;
        make_loader_plan<INSTS>(m, INSTS, VW, EB, args.n_in, 1, m.blk_vec, t - kConsumerThreads, &lp);
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kRows;
            issue_stage<INSTS>(lp, INSTS, X + n0 * args.n_in, stage_limit(n0, row_end, args.n_in, EB),
                               lds + (s % kStages) * kStageBytes);
        };
        for (int s = 0; s < kStages - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            wait_vmcnt_upto(min(kStages - 2, nsteps - 1 - s) * INSTS);
            lds_barrier();                                   // stage s ready
            if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
            lds_barrier();                                   // Z written
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // (A) thread -> delta0 and two beta0 values of the tile
    const int d0 = t & (kD0 - 1);
    const int bpair = t >> 6;                              // 0..3
    float k0r[2][kC0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const TW* kp = K0 + (int64_t(d0) * args.b0 + beta0 + 2 * bpair + j) * kC0;   // K0[0][d0][beta][:]
#pragma unroll
        for (int g = 0; g < kC0; ++g) k0r[j][g] = to_f32(kp[g]);
    }
    // (B) thread -> one of two rows, (alpha1, beta1) and a run of 4 delta1:
    // lanes in (alpha1, beta1, run) order store 16-byte vectors that tile
    // the row's slab of Y contiguously
    const int rsub = t >> 7;                               // row within a pair of rows
    const int run = t & 1;
    const int b1 = (t >> 1) & (kB1 - 1);
    const int a1 = (t >> 4) & (kBT - 1);                   // 0..7 within the tile
    const int e10 = run * 4;                               // first delta1 of the run
    float k1r[4][kC1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const TW* kp = K1 + ((int64_t(beta0 + a1) * kD1 + e10 + k) * kB1 + b1) * kC1;   // K1[a][e][b][:]
#pragma unroll
        for (int g = 0; g < kC1; ++g) k1r[k][g] = to_f32(kp[g]);
    }
    const int64_t yoff = int64_t(beta0 + a1) * (kB1 * kD1) + b1 * kD1 + e10;

    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();                                                   // stage s ready
        const unsigned char* xs = lds + (s % kStages) * kStageBytes;
        const int64_t n0 = row_begin + int64_t(s) * kRows;
        const int rows = static_cast<int>(min(int64_t(kRows), row_end - n0));
        // (A) Z[r][beta0][d0] = sum_g K0[0][d0][beta0][g] * X[r][g][d0]
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const TX* xr = reinterpret_cast<const TX*>(xs + r * kC0 * kD0 * EB) + d0;
            float z0 = 0.0f, z1 = 0.0f;
#pragma unroll
            for (int g = 0; g < kC0; ++g) {
                const float x = to_f32(xr[g * kD0]);
                z0 = fmaf(k0r[0][g], x, z0);
                z1 = fmaf(k0r[1][g], x, z1);
            }
            float* zr = zs + (r * kBT + 2 * bpair) * kZPitch + d0;
            zr[0] = z0;
            zr[kZPitch] = z1;
        }
        lds_barrier();                                                   // Z written
        // (B) Y[r][a1][b1][e1] = sum_g K1[a1][e1][b1][g] * Z[r][a1][g * 8 + e1]
#pragma unroll
        for (int r0 = 0; r0 < kRows; r0 += 2) {
            const int r = r0 + rsub;
            const float* zr = zs + (r * kBT + a1) * kZPitch + e10;
            floatx4 y = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < kC1; ++g) {
                const floatx4 z = *reinterpret_cast<const floatx4*>(zr + g * kD1);
#pragma unroll
                for (int k = 0; k < 4; ++k) y[k] = fmaf(k1r[k][g], z[k], y[k]);
            }
            if (r < rows)
                __builtin_nontemporal_store(y, reinterpret_cast<floatx4*>(Y + (n0 + r) * args.n_out + yoff));
        }
    }
}

bool shape_ok(const Shape& s0, const Shape& s1) {
    return s0.a == 1 && s0.c == kC0 && s0.d == kD0 && s0.b % kBT == 0 && s1.a == s0.b && s1.b == kB1 &&
           s1.c == kC1 && s1.d == kD1;
}

template <typename TX, typename TW>
ks_status_t launch_typed(const Shape& s0, const Shape& s1, const void* W0, const void* W1, const void* X,
                         float* Y, int64_t batch, hipStream_t stream, int num_cus) {
    FusedArgs args;
    args.b0 = s0.b;
    args.n_in = s0.n_in;
    args.n_mid = s0.n_out;
    args.n_out = s1.n_out;
    args.batch = batch;
    args.n_tiles = s0.b / kBT;
    // about one resident wave of workgroups (two per compute unit)
    const int64_t steps_total = (batch + kRows - 1) / kRows;
    const int64_t splits = std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) * 2 / args.n_tiles);
    const int64_t steps = std::max<int64_t>(1, (steps_total + splits - 1) / splits);
    args.rows_per_split = static_cast<int>(steps * kRows);
    const int64_t nsplit = (batch + args.rows_per_split - 1) / args.rows_per_split;
    const int64_t blocks = nsplit * args.n_tiles;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const size_t lds = size_t(kStages) * (kInsts * int(sizeof(TX)) / 4) * 1024 +
                       size_t(kRows) * kBT * kZPitch * sizeof(float);
    return launch_kernel(fused_pair_kernel<TX, TW>, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads),
                         lds, stream, static_cast<const TX*>(X), static_cast<const TW*>(W0),
                         static_cast<const TW*>(W1), Y, args);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool fused_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1) {
    if (wt0 != wt1) return false;
    if (!(xt == kF32 || xt == kBF16)) return false;
    if (!shape_ok(s0, s1)) return false;
    // the loader addresses a stage with 32-bit byte offsets
    return int64_t(kRows) * s0.n_in * elem_bytes(xt) < (int64_t(1) << 31);
}

ks_status_t launch_fused_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                              const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                              int num_cus) {
    if (!fused_pair_supports(s0, s1, xt, wt0, wt1)) return KS_ERR_UNSUPPORTED;
    if (!aligned16(X)) return KS_ERR_UNSUPPORTED;
    if (xt == kF32 && wt0 == kF32) return launch_typed<float, float>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kBF16 && wt0 == kBF16) return launch_typed<bf16_t, bf16_t>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kF32 && wt0 == kBF16) return launch_typed<float, bf16_t>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
