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
// Workgroup: BT consecutive beta0 (= alpha1) values (32, 16 or 8, the
// largest that divides b0) and a range of rows; one loader wave streams whole
// rows of X into an LDS ring (ks_stream.h), each row followed by 32 bytes of
// padding so that the four rows a matrix-core instruction reads start in
// different banks; the b0 / BT workgroups that share rows run on the same
// XCD, so X is fetched from HBM once and served to the others from L2. Per
// stage of 4 rows, eight consumer waves
//  (A) compute Z[r][beta0][delta0] into LDS on the matrix cores: for a fixed
//      delta0 it is a (rows x c0) by (c0 x beta0) product, and the 16-block
//      4x4x1 fp32 MFMA does 16 such delta0 at once (weights in registers),
//  (B) compute Y[r][alpha1][beta1][delta1] of the previous stage from the
//      other Z buffer on the VALU: runs of 4 delta1 per thread (c1 FMAs per
//      value, weights in registers), stored as 16-byte vectors.
// One LDS barrier per stage separates the two. A wide tile (BT = 32 for
// GPT-2-medium's b0 = 64) cuts the L2 re-reads of X to b0 / BT per row and
// keeps more X bytes in flight per byte of Y than two narrow workgroups
// per compute unit would.
// Z never leaves the chip: the pair moves |X| + |Y| + weights through HBM
// instead of |X| + 2|Z| + |Y|.
//
// Alignment. X and Y need only be aligned to their element size. When X
// starts xshift elements past a 16-byte boundary, the loader streams the
// 16-byte granules that cover each row, from the boundary below it (a
// granule never crosses a page, so the extra bytes are always readable), one
// granule more per row (it lands in the row's padding), and the consumers
// read every element xshift places further on. When Y is not 16-byte
// aligned, phase B stores single elements.

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
constexpr int kRows = 4;                   // rows per stage
constexpr int kXPadBytes = 32;             // LDS pad after each row of X: rows start 8 banks apart
constexpr int kZPitch = kD0 + 8;           // Z pitch per beta0 (floats): beta0 neighbours 8 banks apart
constexpr int kZBufs = 2;                  // Z double buffer: phase B of stage s - 1 runs beside phase A of stage s
constexpr int kFusedConsumers = 8;         // consumer waves per workgroup
constexpr int kFusedThreads = kFusedConsumers * 64 + 64;   // + one loader wave

// Geometry of a tile of BT beta0 (= alpha1) values.
template <int BT>
struct FusedTile {
    static constexpr int kZRow = BT * kZPitch + 8;       // Z pitch per row (floats): rows 8 banks apart
    static constexpr int kZFloats = kRows * kZRow;       // one Z buffer
    static constexpr int kSetsPerWave = BT / kFusedConsumers;   // phase A: groups of 4 beta0 per wave
    static constexpr int kRowsPerPass = kFusedConsumers * 64 / (BT * kB1 * 2);   // phase B: rows per pass
    static_assert(BT == 8 || BT == 16 || BT == 32, "tile widths");
    static_assert(kRowsPerPass >= 1 && kRows % kRowsPerPass == 0 && (kZPitch * 4) % 16 == 0 &&
                      (kZRow * 4) % 16 == 0,
                  "phase B covers whole rows per pass, Z in 16-byte runs");
    // phase A: wave w takes delta0 in [16 (w % 4), +16) and the beta0 groups
    // [(w / 4) * kSetsPerWave * 4, +kSetsPerWave * 4)
    static_assert(kRows == 4 && kD0 == 64 && kFusedConsumers == 8 && (kFusedConsumers / 4) * kSetsPerWave * 4 == BT,
                  "phase A: 4x4 MFMA blocks of rows x beta0, 16 delta0 per block group");
};

// Loader instructions (1 KB each) for one stage of rows of elem_bytes-wide
// elements with kXPadBytes after each row.
constexpr int stage_insts(int eb) { return (kRows * (kC0 * kD0 * eb + kXPadBytes) + 1023) / 1024; }
constexpr int stage_bytes(int eb) { return stage_insts(eb) * 1024; }
constexpr int kStagesF32 = 3;              // LDS ring depth for fp32 rows
constexpr int kStagesBF16 = 4;             // ... and for bf16 rows (half the bytes)
constexpr int stages_for(int eb) { return eb == 4 ? kStagesF32 : kStagesBF16; }
constexpr size_t fused_lds_bytes(int eb, int bt) {
    return size_t(stages_for(eb)) * stage_bytes(eb) + size_t(kZBufs) * kRows * (bt * kZPitch + 8) * sizeof(float);
}

struct FusedArgs {
    int b0;                 // beta0 extent (= alpha1 extent)
    int64_t n_in, n_mid, n_out;
    int64_t batch;
    int n_tiles;            // b0 / BT
    int rows_per_split;     // multiple of kRows
    int xshift;             // elements from the 16-byte boundary below X to X (the same in every row)
};

// The byte limit of issue_stage when rows start xshift elements past a
// 16-byte boundary: the granule holding the last elements of the stage's last
// row is one past the usual limit.
__device__ __forceinline__ uint32_t shifted_limit(uint32_t limit, int xshift) {
    return (xshift == 0 || limit > kNoVector - 16u) ? limit : limit + 16u;
}

// kYVec: Y is 16-byte aligned (vector stores in phase B); BT: beta0 per tile.
template <typename TX, typename TW, bool kYVec, int BT>
__global__ __launch_bounds__(kFusedThreads) void fused_pair_kernel(const TX* __restrict__ X,
                                                                   const TW* __restrict__ K0,
                                                                   const TW* __restrict__ K1,
                                                                   float* __restrict__ Y, FusedArgs args) {
    constexpr int EB = int(sizeof(TX));
    constexpr int VW = 16 / EB;
    constexpr int INSTS = stage_insts(EB);
    constexpr int kStageBytes = stage_bytes(EB);
    constexpr int kStages = stages_for(EB);
    constexpr int kRowBytes = kC0 * kD0 * EB + kXPadBytes;   // LDS pitch of a row of X
    using Tile = FusedTile<BT>;
    constexpr int kZRow = Tile::kZRow;
    constexpr int kZFloats = Tile::kZFloats;
    constexpr int kSetsPerWave = Tile::kSetsPerWave;
    constexpr int kRowsPerPass = Tile::kRowsPerPass;
    extern __shared__ __align__(16) unsigned char lds[];
    float* const zs = reinterpret_cast<float*>(lds + kStages * kStageBytes);   // kZBufs x [kRows][BT][kZPitch]

    const int t = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    const int beta0 = tile * BT;                           // first beta0 (= alpha1) of the tile

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kRows - 1) / kRows);

    if (t >= kFusedConsumers * 64) {
        // ------------------------------------------------------ loader wave
        StageMap m;
        m.rows = kRows;
        m.blocks = 1;
        // one whole row of X, and the granule past it when X is not 16-byte
        // aligned (it takes the first vector of the row's padding)
        const int extra = args.xshift != 0 ? 1 : 0;
        m.blk_vec = kC0 * kD0 / VW + extra;
        m.pad_vec = kXPadBytes / 16 - extra;
        m.row_vec = m.blk_vec + m.pad_vec;
        m.gstride = 0;
        LoaderPlan<INSTS> lp;
        make_loader_plan<INSTS>(m, INSTS, VW, EB, args.n_in, 1, m.blk_vec, t - kFusedConsumers * 64, &lp);
        const TX* xbase = X - args.xshift;                 // 16-byte aligned
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kRows;
            issue_stage<INSTS>(lp, INSTS, xbase + n0 * args.n_in,
                               shifted_limit(stage_limit(n0, row_end, args.n_in, EB), args.xshift),
                               lds + (s % kStages) * kStageBytes);
        };
        for (int s = 0; s < kStages - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s <= nsteps; ++s) {
            if (s < nsteps) wait_vmcnt_upto(min(kStages - 2, nsteps - 1 - s) * INSTS);
            lds_barrier();                                   // stage s ready, Z of stage s - 1 written
            if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // Phase A is a batched 4x4 outer product on the matrix cores: in
    // v_mfma_f32_4x4x1f32 lane l belongs to block l / 4, supplies row l % 4
    // of that block's A column and column l % 4 of its B row, and receives
    // D[i][l % 4] of its block in accumulator register i. One instruction
    // per gamma and group of 4 output columns.
    const int lane = t & 63;
    const int wave = t >> 6;
    const int q = lane & 3;                                // A: row; B and D: column within a group of 4
    // (A) block = delta0, A = X[row][gamma0][delta0], B = K0[0][delta0][beta0][gamma0];
    // wave w -> delta0 in [16 (w % 4), 16 (w % 4) + 16) and kSetsPerWave
    // groups of 4 beta0, all kRows rows
    const int a_d0 = 16 * (wave & 3) + (lane >> 2);        // delta0 of this lane's block
    const int a_b0 = (wave >> 2) * kSetsPerWave * 4;       // first beta0 (within the tile) of the wave
    float k0r[kSetsPerWave][kC0];
#pragma unroll
    for (int j = 0; j < kSetsPerWave; ++j) {
        const TW* kp = K0 + (int64_t(a_d0) * args.b0 + beta0 + a_b0 + 4 * j + q) * kC0;   // K0[0][d0][beta][:]
#pragma unroll
        for (int g = 0; g < kC0; ++g) k0r[j][g] = to_f32(kp[g]);
    }

    // (A) Z[r][beta0][d0] = sum_g K0[0][d0][beta0][g] * X[r][g][d0] for stage s
    auto phase_a = [&](int s, float* zb) {
        const unsigned char* xs = lds + (s % kStages) * kStageBytes;
#pragma unroll
        for (int rg = 0; rg < kRows; rg += 4) {
            const TX* xa = reinterpret_cast<const TX*>(xs + (rg + q) * kRowBytes) + args.xshift + a_d0;
            floatx4 z[kSetsPerWave];
#pragma unroll
            for (int j = 0; j < kSetsPerWave; ++j) z[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < kC0; ++g) {
                const float x = to_f32(xa[g * kD0]);
#pragma unroll
                for (int j = 0; j < kSetsPerWave; ++j) z[j] = __builtin_amdgcn_mfma_f32_4x4x1f32(x, k0r[j][g], z[j], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < kSetsPerWave; ++j) {
                float* zw = zb + rg * kZRow + (a_b0 + 4 * j + q) * kZPitch + a_d0;   // lane's beta0 and delta0
#pragma unroll
                for (int i = 0; i < 4; ++i) zw[i * kZRow] = z[j][i];
            }
        }
    };

    // one barrier per stage: phase A of stage s and phase B of stage s - 1
    // share an iteration, on alternate Z buffers
    auto pipeline = [&](auto&& phase_b) {
        for (int s = 0; s <= nsteps; ++s) {
            lds_barrier();                                   // stage s ready, Z of stage s - 1 written
            if (s < nsteps) phase_a(s, zs + (s & 1) * kZFloats);
            if (s > 0) phase_b(s - 1, zs + ((s - 1) & 1) * kZFloats);
        }
    };

    // (B) thread -> one row of a pass, (alpha1, beta1) and a run of 4 delta1:
    // lanes in (alpha1, beta1, run) order store 16-byte vectors that tile
    // the row's slab of Y contiguously
    const int rsub = t / (BT * kB1 * 2);               // row within a pass
    const int run = t & 1;
    const int b1 = (t >> 1) & (kB1 - 1);
    const int a1 = (t >> 4) & (BT - 1);                // alpha1 within the tile
    const int e10 = run * 4;                           // first delta1 of the run
    float k1r[4][kC1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const TW* kp = K1 + ((int64_t(beta0 + a1) * kD1 + e10 + k) * kB1 + b1) * kC1;   // K1[a][e][b][:]
#pragma unroll
        for (int g = 0; g < kC1; ++g) k1r[k][g] = to_f32(kp[g]);
    }
    const int64_t yoff = int64_t(beta0 + a1) * (kB1 * kD1) + b1 * kD1 + e10;
    auto phase_b = [&](int s, const float* zb) {
        const int64_t n0 = row_begin + int64_t(s) * kRows;
        const int rows = static_cast<int>(min(int64_t(kRows), row_end - n0));
#pragma unroll
        for (int r0 = 0; r0 < kRows; r0 += kRowsPerPass) {
            const int r = r0 + rsub;
            const float* zr = zb + r * kZRow + a1 * kZPitch + e10;
            floatx4 y = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < kC1; ++g) {
                const floatx4 z = *reinterpret_cast<const floatx4*>(zr + g * kD1);
#pragma unroll
                for (int k = 0; k < 4; ++k) y[k] = fmaf(k1r[k][g], z[k], y[k]);
            }
            if (r < rows) {
                float* yr = Y + (n0 + r) * args.n_out + yoff;
                if constexpr (kYVec) {
                    __builtin_nontemporal_store(y, reinterpret_cast<floatx4*>(yr));
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(y[k], yr + k);
                }
            }
        }
    };
    pipeline(phase_b);
}

bool shape_ok(const Shape& s0, const Shape& s1) {
    return s0.a == 1 && s0.c == kC0 && s0.d == kD0 && s0.b % 8 == 0 && s1.a == s0.b && s1.b == kB1 &&
           s1.c == kC1 && s1.d == kD1;
}

template <typename TX, typename TW, int BT>
ks_status_t launch_tile(const Shape& s0, const Shape& s1, const void* W0, const void* W1, const void* X,
                        float* Y, int64_t batch, hipStream_t stream, int num_cus) {
    FusedArgs args;
    args.b0 = s0.b;
    args.n_in = s0.n_in;
    args.n_mid = s0.n_out;
    args.n_out = s1.n_out;
    args.batch = batch;
    args.n_tiles = s0.b / BT;
    args.xshift = static_cast<int>((reinterpret_cast<uintptr_t>(X) & 15u) / sizeof(TX));
    // about one resident wave of workgroups (as many per compute unit as fit its 160 KB of LDS)
    const size_t lds = fused_lds_bytes(int(sizeof(TX)), BT);
    const int per_cu = std::max(1, std::min(4, int((160 * 1024) / lds)));
    const int64_t steps_total = (batch + kRows - 1) / kRows;
    const int64_t splits = std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) * per_cu / args.n_tiles);
    const int64_t steps = std::max<int64_t>(1, (steps_total + splits - 1) / splits);
    args.rows_per_split = static_cast<int>(steps * kRows);
    const int64_t nsplit = (batch + args.rows_per_split - 1) / args.rows_per_split;
    const int64_t blocks = nsplit * args.n_tiles;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const bool y_vec = (reinterpret_cast<uintptr_t>(Y) & 15u) == 0;
    auto kernel = y_vec ? fused_pair_kernel<TX, TW, true, BT> : fused_pair_kernel<TX, TW, false, BT>;
    return launch_kernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kFusedThreads), lds, stream,
                         static_cast<const TX*>(X), static_cast<const TW*>(W0), static_cast<const TW*>(W1), Y, args);
}

// The widest tile that divides b0: 32 beta0 per workgroup on GPT-2-medium's
// b0 = 64 (fp32 64 vs 72 us, bf16 61 vs 68 us against 8 beta0 and four
// compute waves, measured A/B in one process).
template <typename TX, typename TW>
ks_status_t launch_typed(const Shape& s0, const Shape& s1, const void* W0, const void* W1, const void* X,
                         float* Y, int64_t batch, hipStream_t stream, int num_cus) {
    if (s0.b % 32 == 0) return launch_tile<TX, TW, 32>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    if (s0.b % 16 == 0) return launch_tile<TX, TW, 16>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    return launch_tile<TX, TW, 8>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
}

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
    // X and Y aligned to their element size (checked by the caller); rows
    // are whole 16-byte granules apart, so every row has X's misalignment
    if ((reinterpret_cast<uintptr_t>(X) % elem_bytes(xt)) != 0 || (reinterpret_cast<uintptr_t>(Y) & 3u) != 0 ||
        (s0.n_in * elem_bytes(xt)) % 16 != 0)
        return KS_ERR_UNSUPPORTED;
    if (xt == kF32 && wt0 == kF32) return launch_typed<float, float>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kBF16 && wt0 == kBF16) return launch_typed<bf16_t, bf16_t>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kF32 && wt0 == kBF16) return launch_typed<float, bf16_t>(s0, s1, W0, W1, X, Y, batch, stream, num_cus);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
