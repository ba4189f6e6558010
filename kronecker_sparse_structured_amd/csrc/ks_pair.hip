// ks_pair.hip -- two butterfly-type KS factors in one launch when the second
// one mixes the digit just below the one the first mixes.
//
// Butterfly layers are chains of KS factors (KS abstract page,
// taxoreview.com "dblp:303/4794", first paragraph). Take F = (a, 16, 16, d)
// with d = 16 e, followed by G = (16 a, 16, 16, e): two consecutive factors
// of a radix-16 butterfly (the last two, e = 1, are ks_slab.hip's). Write
// F's delta as h * e + t (h < 16, t < e). F maps
//     X[alpha][gamma][h][t]  ->  Z[alpha][beta][h][t]
// (a 16 x 16 block per (alpha, h, t)), and G reads Z as
// Z[alpha' = 16 alpha + beta][gamma' = h][delta' = t], mapping it to
//     Y[alpha'][beta'][t] = Y[alpha][beta][beta'][t]
// (a 16 x 16 block per (alpha', t)). So for a fixed (alpha, t) the 256
// values X[alpha][.][.][t] determine exactly the 256 values
// Y[alpha][.][.][t], at the same places of the row, through 16 + 16 blocks:
// a closed group, e elements apart. A tile takes 4 consecutive t, whose
// values lie in 16-byte runs, e * 4 bytes apart: it reads and writes each
// row of its part once and needs 32 blocks of each factor (128 KB of fp32),
// which the four compute waves hold in registers. The intermediate Z never
// leaves the chip: the pair moves |X| + |Y| through HBM instead of
// |X| + 2|Z| + |Y|.
//
// Workgroup: one loader wave streams the tile's part of 16 rows (64 KB) into
// one of two LDS stages with global_load_lds_dwordx4; four compute waves,
// per stage,
//  (A) compute Z in place on the matrix cores: for a fixed (h, t),
//      Z[rows][beta] = X[rows][gamma] (16 x 16) times the block's transpose;
//      wave w takes h = 4w .. 4w + 3, and one 16-byte LDS read gives the A
//      operands of the 4 t of the tile at once;
//  (B) after an LDS barrier, compute Y in place the same way: for a fixed
//      (beta, t), Y[rows][beta'] = Z[rows][beta][h] (16 x 16) times G's block
//      transposed; wave w takes beta = 4w .. 4w + 3;
//  (C) after another barrier, store the stage as 16-byte vectors.
// Each wave reads and writes only LDS places of its own h (A) or beta (B),
// so working in place needs no barrier inside a phase.
//
// LDS layout of a stage, in 16-byte vectors: row r, index x (gamma, then
// beta), vector v (one run of the 4 t) at r * 273 + x * 17 + v. The padding
// (17 = 16 + 1 per index, 273 = 16 * 17 + 1 per row) puts the 16 lanes that
// one access pattern spreads over rows, x or v into 16 different 16-byte bank
// groups, for all four patterns (reads and writes of both phases), and keeps
// every address a per-lane base plus a constant.
//
// X and Y must be 16-byte aligned with 16-byte rows; the chain planner runs
// the two factors one at a time otherwise.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kN = 16;                 // b = c of both factors; the digits mixed
constexpr int kT = 4;                  // t per tile: one 16-byte run of fp32
constexpr int kR = 16;                 // rows per stage: one MFMA M tile
constexpr int kXVec = kN + 1;          // LDS vectors per index x (16 runs + 1 pad)
constexpr int kRowVec = kN * kXVec + 1; // LDS vectors per row (273)
constexpr int kStageVec = kR * kRowVec;
constexpr int kStageInsts = (kStageVec + 63) / 64;  // loader instructions per stage (69)
constexpr int kStageBytes = kStageInsts * 1024;     // 69 KB
constexpr int kStages = 2;
constexpr int kThreads = kStreamThreads;          // 4 compute waves + 1 loader wave

struct PairArgs {
    int a, d, e;             // F = (a, 16, 16, d), d = 16 e; G = (16 a, 16, 16, e)
    int64_t n;               // row width of X, Z and Y: 256 a e
    int64_t batch;
    int tblocks;             // e / kT
    int n_tiles;             // a * tblocks
    int rows_per_split;      // a multiple of kR
};

// LDS vector index (within a stage) of row r, index x, vector v.
__device__ __forceinline__ int lds_vec(int r, int x, int v) { return r * kRowVec + x * kXVec + v; }

template <typename TW>
__global__ __launch_bounds__(kThreads) void strided_pair_kernel(const float* __restrict__ X,
                                                                const TW* __restrict__ KF,
                                                                const TW* __restrict__ KG,
                                                                float* __restrict__ Y, PairArgs args) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int t = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    // the t-blocks of one alpha are neighbours: those sharing cache lines of
    // X and Y run on the same XCD
    const int alpha = tile / args.tblocks;
    const int t0 = (tile - alpha * args.tblocks) * kT;
    const int64_t d = args.d, e = args.e;
    const int64_t g0 = int64_t(alpha) * kN * d + t0;   // the tile's first element in a row

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kR - 1) / kR);

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        // instruction i fills LDS vectors [64 i, 64 i + 64) of a stage; a
        // lane whose vector is padding (or past the stage) loads the stage's
        // first run again, which nothing reads
        const int lane = t - kConsumerThreads;
        uint32_t off[kStageInsts];
#pragma unroll
        for (int i = 0; i < kStageInsts; ++i) {
            const int q = 64 * i + lane;
            const int r = q / kRowVec, u = q - r * kRowVec, x = u / kXVec, v = u - x * kXVec;
            off[i] = (r < kR && x < kN && v < kN) ? static_cast<uint32_t>((r * args.n + x * d + v * e) * 4) : 0u;
        }
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const uint32_t limit = stage_limit(n0, row_end, args.n, 4);
            const char* base = reinterpret_cast<const char*>(X + n0 * args.n + g0);
            unsigned char* st = lds + (s % kStages) * kStageBytes;
#pragma unroll
            for (int i = 0; i < kStageInsts; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (off[i] < limit ? off[i] : 0u)),
                                                 st + 1024 * i, 16, 0, 0);
        };
        for (int s = 0; s < kStages && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // stage s has landed once at most the next stage's loads are in
            // flight (loads complete in order; 63 is vmcnt's largest count,
            // less than a stage, so this waits a few loads longer)
            if (s + 1 < nsteps) wait_vmcnt<63>();
            else wait_vmcnt<0>();
            lds_barrier();                                   // stage s ready
            lds_barrier();                                   // Z written
            lds_barrier();                                   // Y written
            lds_barrier();                                   // stage s read out
            if (s + kStages < nsteps) issue(s + kStages);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + i][l % 16] in register i.
    const int w = t >> 6;
    const int lane = t & 63;
    const int col = lane & 15;      // A: row; B and D: output column
    const int grp = lane >> 4;      // A and B: k within a step; D: group of 4 rows
    // (A) h = 4w + hh: B = K_F[alpha][h e + t0 + tt][beta = col][gamma = 4 ks + grp]
    float kf[4][kT][4];
    // (B) beta = 4w + bb: B = K_G[16 alpha + beta][t0 + tt][beta' = col][h = 4 ks + grp]
    float kg[4][kT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
            const int64_t delta = int64_t(4 * w + q) * e + t0 + tt;
            const TW* fp = KF + ((int64_t(alpha) * d + delta) * kN + col) * kN + grp;
            const TW* gp = KG + ((int64_t(kN * alpha + 4 * w + q) * e + t0 + tt) * kN + col) * kN + grp;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kf[q][tt][ks] = to_f32(fp[4 * ks]);
                kg[q][tt][ks] = to_f32(gp[4 * ks]);
            }
        }
    }

    for (int s = 0; s < nsteps; ++s) {
        floatx4* st = reinterpret_cast<floatx4*>(lds + (s % kStages) * kStageBytes);
        lds_barrier();                                                   // stage s ready
        // (A) Z[r][beta][h][tt] = sum_gamma K_F[alpha][h e + t0 + tt][beta][gamma] X[r][gamma][h][tt]
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const int h = 4 * w + hh;
            floatx4 z[kT];
#pragma unroll
            for (int tt = 0; tt < kT; ++tt) z[tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const floatx4 xv = st[lds_vec(col, 4 * ks + grp, h)];   // the 4 t of X[col][gamma][h]
#pragma unroll
                for (int tt = 0; tt < kT; ++tt)
                    z[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[tt], kf[hh][tt][ks], z[tt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st[lds_vec(4 * grp + i, col, h)] = floatx4{z[0][i], z[1][i], z[2][i], z[3][i]};
        }
        lds_barrier();                                                   // Z written
        // (B) Y[r][beta][beta'][tt] = sum_h K_G[16 alpha + beta][t0 + tt][beta'][h] Z[r][beta][h][tt]
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int beta = 4 * w + bb;
            floatx4 y[kT];
#pragma unroll
            for (int tt = 0; tt < kT; ++tt) y[tt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const floatx4 zv = st[lds_vec(col, beta, 4 * ks + grp)];   // the 4 t of Z[col][beta][h]
#pragma unroll
                for (int tt = 0; tt < kT; ++tt)
                    y[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[tt], kg[bb][tt][ks], y[tt], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st[lds_vec(4 * grp + i, beta, col)] = floatx4{y[0][i], y[1][i], y[2][i], y[3][i]};
        }
        lds_barrier();                                                   // Y written
        // (C) thread t stores, in every row j, the run of index x = t / 16 and
        // vector v = t % 16: Y[j][alpha][beta = x][beta' = v][t0 ..]; four
        // rows at a time (their LDS reads, then their stores), the stage
        // released once the last rows have been read
        {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const int rows = static_cast<int>(min(int64_t(kR), row_end - n0));
            const int x = t >> 4, v = t & 15;
            float* yrun = Y + n0 * args.n + g0 + x * d + v * e;
#pragma unroll
            for (int j0 = 0; j0 < kR; j0 += 4) {
                floatx4 y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = st[lds_vec(j0 + j, x, v)];
                if (j0 + 4 == kR) lds_barrier();                         // stage s read out
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j0 + j < rows)
                        __builtin_nontemporal_store(y[j], reinterpret_cast<floatx4*>(yrun + (j0 + j) * args.n));
            }
        }
    }
}

bool shape_ok(const Shape& s0, const Shape& s1) {
    return s0.b == kN && s0.c == kN && s0.d % (kN * kT) == 0 && s1.a == int64_t(s0.a) * kN && s1.b == kN &&
           s1.c == kN && s1.d * kN == s0.d;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename TW>
ks_status_t launch_typed(const Shape& s0, const void* W0, const void* W1, const void* X, float* Y, int64_t batch,
                         hipStream_t stream, int num_cus) {
    PairArgs args;
    args.a = s0.a;
    args.d = s0.d;
    args.e = s0.d / kN;
    args.n = s0.n_in;
    args.batch = batch;
    args.tblocks = args.e / kT;
    args.n_tiles = args.a * args.tblocks;
    // one workgroup per compute unit (two 64 KB stages), equal row shares
    const int64_t steps_total = (batch + kR - 1) / kR;
    const int64_t splits = std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) / args.n_tiles);
    const int64_t steps = std::max<int64_t>(1, (steps_total + splits - 1) / splits);
    args.rows_per_split = static_cast<int>(steps * kR);
    const int64_t nsplit = (batch + args.rows_per_split - 1) / args.rows_per_split;
    const int64_t blocks = nsplit * args.n_tiles;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    return launch_kernel(strided_pair_kernel<TW>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                         size_t(kStages) * kStageBytes, stream, static_cast<const float*>(X),
                         static_cast<const TW*>(W0), static_cast<const TW*>(W1), Y, args);
}

}  // namespace

// e at most this: a tile's 16-byte runs are e * 4 bytes apart, so they fill
// the cache lines they touch when e = 4 and half of them when e = 8. Beyond
// that the pair loses to two launches (measured on 4,096 rows of 65,536,
// fp32, fused against one launch per factor: e = 4 0.40 against 0.77 ms,
// e = 8 0.54 against 0.75 ms, e = 16 0.91 against 0.80 ms, e = 256 1.60
// against 0.83 ms): each CU's outstanding line misses then carry too few
// useful bytes.
constexpr int kMaxE = 8;

bool strided_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1) {
    if (wt0 != wt1 || xt != kF32 || !(wt0 == kF32 || wt0 == kBF16)) return false;
    if (!shape_ok(s0, s1) || s1.d > kMaxE) return false;
    // the loader addresses a stage with 32-bit byte offsets; tiles per launch
    return int64_t(kR) * s0.n_in * 4 < (int64_t(1) << 31) && int64_t(s0.a) * (s0.d / kN / kT) < (int64_t(1) << 24);
}

bool strided_pair_aligned(const void* X, const void* Y) { return aligned16(X) && aligned16(Y); }

ks_status_t launch_strided_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                                const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                                int num_cus) {
    if (!strided_pair_supports(s0, s1, xt, wt0, wt1) || !strided_pair_aligned(X, Y)) return KS_ERR_UNSUPPORTED;
    if (wt0 == kF32) return launch_typed<float>(s0, W0, W1, X, Y, batch, stream, num_cus);
    return launch_typed<bf16_t>(s0, W0, W1, X, Y, batch, stream, num_cus);
}

}  // namespace ks
