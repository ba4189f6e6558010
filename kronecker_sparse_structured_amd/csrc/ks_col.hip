// ks_col.hip -- one KS factor with square 16 x 16 or 32 x 32 blocks and
// d >= 16, computed in place in LDS.
//
// Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
//                                    * X[n][alpha][gamma][delta]
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph). With
// b = c = N and many deltas, a row's part for one alpha and a run of DT
// deltas is N segments of DT elements, d apart, in X and in Y alike: the
// place X[.][alpha][x][delta] holds gamma = x before the product and
// beta = x after it. A workgroup owns (alpha, DT deltas), streams 16 rows of
// its part of X per stage into an LDS ring, and its four compute waves
// overwrite each stage with Y in place: a wave owns whole 16-byte vectors
// (4 deltas) of the tile, reads all N gammas of its deltas for 16 rows
// (one 16-byte read gives the A operands of four deltas) and writes all N
// betas back to the same vectors. A storer wave writes stage s - 1 to Y
// while stage s computes and the loader wave fills stages s + 1 and s + 2,
// so one LDS barrier per stage separates them all.
//
// Stage layout, in 16-byte vectors: row r, index x (gamma, then beta),
// vector v (deltas 4v .. 4v + 3 of the tile) at r * RP + x * XP + v with
// XP = DT / 4 + 1 and RP = N * XP + 1, both odd, so the 16 rows (A reads) or
// the 16 betas (D writes) that one instruction touches fall in 16 different
// 16-byte bank groups. X is fp32 (the stage is rewritten with fp32 Y); X and
// Y must be 16-byte aligned with 16-byte rows.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kR = 16;                                  // rows per stage: one MFMA M tile
constexpr int kColThreads = kStreamThreads + 64;        // 4 compute waves, loader, storer
constexpr int kStoreBatch = 8;                          // storer: vectors per lane in flight

template <int N>
struct ColShape {
    static constexpr int DT = N == 16 ? 32 : 16;        // deltas per tile (128 / 64-byte runs)
    static constexpr int VPT = DT / 4;                  // 16-byte vectors per segment
    static constexpr int VPW = VPT / 4;                 // vectors per compute wave
    static constexpr int XP = VPT + 1;                  // LDS vectors per index x
    static constexpr int RP = N * XP + 1;               // LDS vectors per row
    static constexpr int STAGE_VEC = kR * RP;
    static constexpr int INSTS = (STAGE_VEC + 63) / 64; // loader instructions per stage
    static constexpr int STAGE_BYTES = INSTS * 1024;
    static constexpr int STAGES = (150 * 1024) / STAGE_BYTES;   // ring depth
    static constexpr int NT = N / 16;                   // MFMA N tiles (betas)
    static constexpr int KS = N / 4;                    // MFMA K steps (gammas)
    static constexpr int YVEC = kR * N * VPT;           // Y vectors of a stage
    static_assert(VPW >= 1 && VPW * 4 == VPT, "whole vectors per wave");
    static_assert(STAGES >= 3 && (STAGES - 3) * INSTS <= 63, "ring depth and exact loader waits");
    static_assert(YVEC % (64 * kStoreBatch) == 0, "storer batches");
};

struct ColArgs {
    int a, d;
    int64_t n_in;            // = n_out = a * N * d
    int64_t batch;
    int tiles_delta;         // d / DT
    int n_tiles;             // a * tiles_delta
    int rows_per_split;      // a multiple of kR
};

template <int N, typename TW>
__global__ __launch_bounds__(kColThreads) void col_kernel(const float* __restrict__ X, const TW* __restrict__ K,
                                                          float* __restrict__ Y, ColArgs args) {
    using S = ColShape<N>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int t = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    // the delta tiles of one alpha are neighbours, on one XCD
    const int alpha = tile / args.tiles_delta;
    const int delta0 = (tile - alpha * args.tiles_delta) * S::DT;
    const int64_t d = args.d;
    const int64_t g0 = int64_t(alpha) * N * d + delta0;     // the tile's first element in a row

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kR - 1) / kR);
    auto stage = [&](int s) { return reinterpret_cast<floatx4*>(lds + (s % S::STAGES) * S::STAGE_BYTES); };

    if (t >= kStreamThreads) {
        // ------------------------------------------------------ storer wave
        // stage s - 1 during step s: every vector, 16-byte stores; lane l
        // takes the vectors q = l + 64 j of the stage in Y's order (row,
        // beta, vector), so one instruction writes whole 128- or 64-byte runs
        __builtin_amdgcn_s_setprio(3);
        const int lane = t & 63;
        auto store_stage = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const int rows = static_cast<int>(min(int64_t(kR), row_end - n0));
            const floatx4* st = stage(s);
            float* ybase = Y + n0 * args.n_in + g0;
#pragma unroll
            for (int j0 = 0; j0 < S::YVEC / 64; j0 += kStoreBatch) {
                floatx4 v[kStoreBatch];
#pragma unroll
                for (int j = 0; j < kStoreBatch; ++j) {
                    const int q = lane + 64 * (j0 + j);
                    const int r = q / (N * S::VPT), rem = q - r * (N * S::VPT);
                    const int x = rem / S::VPT, vv = rem - x * S::VPT;
                    v[j] = st[r * S::RP + x * S::XP + vv];
                }
#pragma unroll
                for (int j = 0; j < kStoreBatch; ++j) {
                    const int q = lane + 64 * (j0 + j);
                    const int r = q / (N * S::VPT), rem = q - r * (N * S::VPT);
                    const int x = rem / S::VPT, vv = rem - x * S::VPT;
                    if (r < rows)
                        __builtin_nontemporal_store(
                            v[j], reinterpret_cast<floatx4*>(ybase + r * args.n_in + x * d + 4 * vv));
                }
            }
        };
        for (int s = 0; s < nsteps; ++s) {
            lds_barrier();                                   // stage s ready, stage s - 1 computed
            if (s > 0) store_stage(s - 1);
        }
        lds_barrier();                                       // last stage computed
        store_stage(nsteps - 1);
        return;
    }

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        // instruction i fills LDS vectors [64 i, 64 i + 64) of a stage; a lane
        // whose vector is padding (or past the stage) loads the stage's first
        // vector again, which nothing reads
        const int lane = t - kConsumerThreads;
        uint32_t off[S::INSTS];
#pragma unroll
        for (int i = 0; i < S::INSTS; ++i) {
            const int q = 64 * i + lane;
            const int r = q / S::RP, u = q - r * S::RP, x = u / S::XP, v = u - x * S::XP;
            off[i] = (r < kR && x < N && v < S::VPT) ? static_cast<uint32_t>((r * args.n_in + x * d + 4 * v) * 4) : 0u;
        }
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const uint32_t limit = stage_limit(n0, row_end, args.n_in, 4);
            const char* base = reinterpret_cast<const char*>(X + n0 * args.n_in + g0);
            unsigned char* st = reinterpret_cast<unsigned char*>(stage(s));
#pragma unroll
            for (int i = 0; i < S::INSTS; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (off[i] < limit ? off[i] : 0u)),
                                                 st + 1024 * i, 16, 0, 0);
        };
        // stages 0 .. S-3 up front; at step s the slot of stage s - 2 (stored
        // during step s - 1) takes stage s + S - 2
        for (int s = 0; s < S::STAGES - 2 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // stage s has landed once only the stages issued after it remain
            wait_vmcnt_upto(min(S::STAGES - 3, nsteps - 1 - s) * S::INSTS);
            lds_barrier();                                   // stage s ready, stage s - 1 computed
            if (s + S::STAGES - 2 < nsteps) issue(s + S::STAGES - 2);
        }
        lds_barrier();                                       // last stage computed
        return;
    }

    // ---------------------------------------------------------- consumers
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + i][l % 16] in register i.
    // Wave w owns the vectors w * VPW .. (deltas 4 v + u of the tile).
    const int w = t >> 6;
    const int lane = t & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    float kr[S::VPW][4][S::NT][S::KS];      // B = K[alpha][delta][beta = 16 nt + col][gamma = 4 ks + grp]
#pragma unroll
    for (int vi = 0; vi < S::VPW; ++vi) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int delta = delta0 + 4 * (w * S::VPW + vi) + u;
            const TW* kp = K + ((int64_t(alpha) * d + delta) * N + col) * N + grp;
#pragma unroll
            for (int nt = 0; nt < S::NT; ++nt)
#pragma unroll
                for (int ks = 0; ks < S::KS; ++ks) kr[vi][u][nt][ks] = to_f32(kp[16 * nt * N + 4 * ks]);
        }
    }

    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();                                                   // stage s ready
        floatx4* st = stage(s);
#pragma unroll
        for (int vi = 0; vi < S::VPW; ++vi) {
            const int v = w * S::VPW + vi;
            floatx4 acc[4][S::NT];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int nt = 0; nt < S::NT; ++nt) acc[u][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks) {
                const floatx4 xv = st[col * S::RP + (4 * ks + grp) * S::XP + v];   // 4 deltas of X[col][gamma]
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int nt = 0; nt < S::NT; ++nt)
                        acc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[u], kr[vi][u][nt][ks], acc[u][nt], 0, 0, 0);
            }
#pragma unroll
            for (int nt = 0; nt < S::NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[(4 * grp + i) * S::RP + (16 * nt + col) * S::XP + v] =
                        floatx4{acc[0][nt][i], acc[1][nt][i], acc[2][nt][i], acc[3][nt][i]};
        }
    }
    lds_barrier();                                                       // last stage computed
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rows per workgroup. For 16 x 16 blocks, workgroups of 128 rows (several
// rounds of them) measured best: every delta tile of the same rows is then in
// flight at about the same time, where long workgroups drift apart (on
// 4,096 rows of (1, 16, 16, 4096): 0.46, 0.63, 0.66, 0.64, 0.56 of 8 TB/s at
// 32, 64, 128, 256 and 2,048 rows; (8, 16, 16, 32) on 16,384 rows 0.69 at
// 128). For 32 x 32 blocks one round of workgroups measured best.
constexpr int kRowsPerBlock16 = 128;

int64_t col_splits(const Shape& s, int num_cus) {
    const int dt = s.b == 16 ? ColShape<16>::DT : ColShape<32>::DT;
    return std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) / (int64_t(s.a) * (s.d / dt)));
}

template <int N, typename TW>
ks_status_t launch_nt(const FactorCall& f) {
    using S = ColShape<N>;
    ColArgs args;
    args.a = f.s.a;
    args.d = f.s.d;
    args.n_in = f.s.n_in;
    args.batch = f.batch;
    args.tiles_delta = f.s.d / S::DT;
    args.n_tiles = f.s.a * args.tiles_delta;
    // one workgroup per compute unit, equal row shares
    const int64_t steps_total = (f.batch + kR - 1) / kR;
    int64_t steps;
    if (f.rows_per_block > 0) {
        steps = (f.rows_per_block + kR - 1) / kR;
    } else {
        steps = (steps_total + col_splits(f.s, f.num_cus) - 1) / col_splits(f.s, f.num_cus);
        if (N == 16) steps = std::min<int64_t>(steps, kRowsPerBlock16 / kR);
    }
    steps = std::max<int64_t>(1, std::min(steps, steps_total));
    args.rows_per_split = static_cast<int>(steps * kR);
    const int64_t nsplit = (f.batch + args.rows_per_split - 1) / args.rows_per_split;
    const int64_t blocks = nsplit * args.n_tiles;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    return launch_kernel(col_kernel<N, TW>, dim3(static_cast<unsigned>(blocks)), dim3(kColThreads),
                         size_t(S::STAGES) * S::STAGE_BYTES, f.stream, static_cast<const float*>(f.X),
                         static_cast<const TW*>(f.W), f.Y, args);
}

}  // namespace

bool col_supports(const Shape& s, int xt, int wt) {
    if (xt != kF32 || !(wt == kF32 || wt == kBF16)) return false;
    if (s.b != s.c || !(s.b == 16 || s.b == 32)) return false;
    const int dt = s.b == 16 ? ColShape<16>::DT : ColShape<32>::DT;
    if (s.d % dt != 0) return false;
    // the loader addresses a stage with 32-bit byte offsets
    return int64_t(kR) * s.n_in * 4 < (int64_t(1) << 31);
}

// The planner's rule: the column kernel where a tile is a whole alpha slab
// (d = DT), which it streams as one contiguous run per row. Measured on
// 16,384 rows (fraction of 8 TB/s, column kernel against the tiled
// matrix-core kernel): (8, 16, 16, 32) 0.68 / 0.52, (8, 32, 32, 16) 0.58 /
// 0.49. With several tiles per slab it lost: (2, 16, 16, 128) 0.56 / 0.60,
// (4, 32, 32, 32) 0.47 / 0.52, and the butterfly's (1, 16, 16, 4096) on
// 4,096 rows 0.56 / 0.65.
bool col_preferred(const Shape& s, int xt, int wt) {
    return col_supports(s, xt, wt) && s.d == (s.b == 16 ? ColShape<16>::DT : ColShape<32>::DT);
}

int col_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len) {
    if (!col_supports(s, xt, wt)) return std::snprintf(buf, len, "col: unsupported");
    const int dt = s.b == 16 ? ColShape<16>::DT : ColShape<32>::DT;
    const int stages = s.b == 16 ? ColShape<16>::STAGES : ColShape<32>::STAGES;
    const int kb = s.b == 16 ? ColShape<16>::INSTS : ColShape<32>::INSTS;
    const int64_t tiles = int64_t(s.a) * (s.d / dt);
    const int64_t splits = col_splits(s, num_cus);
    int64_t steps = std::max<int64_t>(1, ((batch + kR - 1) / kR + splits - 1) / splits);
    if (s.b == 16) steps = std::min<int64_t>(steps, kRowsPerBlock16 / kR);
    return std::snprintf(buf, len,
                         "col 16x16x4f32 in place: deltas/tile=%d outputs/tile=%d rows/wg=%lld wgs=%lld "
                         "stages=%d x %d KB storers=1",
                         dt, s.b, static_cast<long long>(steps * kR),
                         static_cast<long long>(tiles * ((batch + steps * kR - 1) / (steps * kR))), stages, kb);
}

ks_status_t launch_col(const FactorCall& f) {
    if (!col_supports(f.s, f.xt, f.wt)) return KS_ERR_UNSUPPORTED;
    if (!aligned16(f.X) || !aligned16(f.Y) || (f.s.n_in * 4) % 16 != 0) return KS_ERR_UNSUPPORTED;
    if (f.s.b == 16) return f.wt == kF32 ? launch_nt<16, float>(f) : launch_nt<16, bf16_t>(f);
    return f.wt == kF32 ? launch_nt<32, float>(f) : launch_nt<32, bf16_t>(f);
}

}  // namespace ks
