// ks_valu.hip -- KS matmul for small blocks (b, c in {4, 8, 16}) on the
// vector ALUs.
//
// Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
//                                    * X[n][alpha][gamma][delta]
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph). With
// b, c <= 16 the contraction is a few fp32 FMAs per output and the op is
// bound by HBM traffic, so the kernel is built to move X and Y exactly once,
// in whole 16-byte vectors, with no permutation pass (the same page, third
// sentence: a fused, output-stationary kernel).
//
// Workgroup: a tile of (alpha, delta) pairs (all beta) and a range of rows.
// One loader wave streams the tile's part of each row of X into a 4-stage
// LDS ring (ks_stream.h); four consumer waves compute and store Y.
//
// Every consumer thread owns NB betas of a FIXED set of (alpha, delta)
// pairs, so its NB x DV x c weights are loaded into registers once and
// reused for every row (weight-stationary, output-stationary). Mappings:
//  * lane mode (d >= 8): lanes run over consecutive delta runs of DV = 4
//    deltas (DV = 1 when d is not a multiple of 4); a thread reads DV
//    consecutive X values per gamma from LDS and stores DV consecutive
//    outputs per beta, so both sides move 16-byte vectors across lanes.
//  * slab mode (d in {1, 2, 4}): a thread owns one alpha and all d deltas;
//    it reads the contiguous c*d slab of X with 16-byte LDS reads and stores
//    NB*d contiguous outputs.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxInsts = 31;       // loader instructions (KB) per stage, at most
constexpr int kTargetVec = 16 * 64; // aim for about 16 KB per stage
constexpr int kLdsPerGroup = 80 * 1024;   // two workgroups per compute unit

// Betas per thread: the largest power of two dividing b whose weights
// (NB * dv * c values) fit in 128 registers for c = 16, 64 otherwise, which
// keeps a thread near 168 VGPRs (three waves per SIMD, two workgroups per
// compute unit). The host planner uses the same rule.
__host__ __device__ constexpr int nb_rule(int b, int c, int dv) {
    const int budget = c == 16 ? 128 : 64;
    int nb = b;
    while (nb > 1 && nb * c * dv > budget) nb /= 2;
    return nb;
}

// Betas per thread for a mapping. In slab mode a thread's outputs are
// nb * d consecutive floats; when that run is longer than one 16-byte
// vector, a wave's store instruction writes vectors 16 * nb * d / 4 bytes
// apart and no instruction covers whole lines. Runs of exactly 4 floats
// (nb = 4 / d; the threads of one alpha share its X slab, an LDS broadcast)
// make consecutive lanes store consecutive vectors. Measured: (256, 4, 4, 4)
// 3.9 against 2.5 TB/s (nb 4 -> 1); with c >= 8, (256, 8, 8, 2) +26 %,
// (128, 8, 8, 4) +14 %, (512, 8, 8, 1) +7 % (bf16 +81 %); with c = 4 and
// d = 2 the register rule was 4 % faster, so it stays.
__host__ __device__ constexpr int nb_pick(int b, int c, int dv, bool lane) {
    const int nb = nb_rule(b, c, dv);
    if (lane) return nb;
    if (dv == 4 && nb == b) return 1;
    if (c >= 8 && dv <= 4 && nb * dv > 4 && b % (4 / dv) == 0) return 4 / dv;
    return nb;
}

struct ValuArgs {
    int a, d;
    int64_t n_in, n_out;
    int64_t batch;
    int at;              // alphas per tile
    int dt;              // deltas per tile
    int tiles_delta;     // delta tiles per alpha tile
    int n_tiles;         // alpha tiles * delta tiles
    int rows_per_split;  // rows per workgroup (a multiple of map.rows), dealt in stages round-robin
    int contiguous;      // 1: the tile spans every delta (alpha slabs); 0: gamma segments
    int insts;           // loader instructions per stage (stage = insts KB of LDS)
    int stages;          // LDS ring depth
    int xcd_remap;       // 1: renumber workgroups so neighbouring tiles share an XCD
    StageMap map;        // LDS layout of one stage
};

template <typename TX, typename TW, int B, int C, int DV, bool LANE, bool ILV>
__global__ __launch_bounds__(kStreamThreads) void valu_kernel(const TX* __restrict__ X,
                                                              const TW* __restrict__ K,
                                                              float* __restrict__ Y,
                                                              ValuArgs args) {
    constexpr int EB = int(sizeof(TX));
    constexpr int VW = 16 / EB;                 // elements per 16-byte vector
    constexpr int NB = ILV ? 1 : nb_pick(B, C, DV, LANE);
    constexpr int G = B / NB;                   // beta groups
    constexpr int P = kConsumerThreads / G;     // delta runs (lane) or alphas (slab) per group
    static_assert(B % NB == 0, "beta groups must divide b");

    extern __shared__ __align__(16) unsigned char lds[];
    const int kStageBytes = args.insts * 1024;
    const int kStages = args.stages;

    const int t = threadIdx.x;
    const int blk = args.xcd_remap ? xcd_logical_block(blockIdx.x, gridDim.x) : int(blockIdx.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    const int ta = tile / args.tiles_delta;
    const int td = tile - ta * args.tiles_delta;
    const int alpha0 = ta * args.at;
    const int delta0 = td * args.dt;
    const int d = args.d;
    const int at_eff = min(args.at, args.a - alpha0);
    const int dt_eff = min(args.dt, d - delta0);
    const int64_t chunk_base = int64_t(alpha0) * C * d + (args.contiguous ? 0 : delta0);

    const int R = args.map.rows;
    // Row blocks are dealt round-robin: stage s of split p covers rows
    // (s nsplit + p) R .., so at any time the workgroups of a tile work on
    // neighbouring rows and HBM sees a few compact regions instead of one
    // stream per workgroup (measured, 16,384 rows: (1, 4, 4, 1024) 107 -> 97
    // us, (512, 8, 8, 1) 134 -> 104 us, every VALU pattern faster).
    const int nsplit = gridDim.x / args.n_tiles;
    const int64_t total_steps = (args.batch + R - 1) / R;
    if (split >= total_steps) return;
    const int nsteps = static_cast<int>((total_steps - split + nsplit - 1) / nsplit);
    auto stage_row = [&](int s) -> int64_t { return (int64_t(s) * nsplit + split) * R; };
    const int row_bytes = args.map.row_vec * 16;
    const int pitch_bytes = (args.map.blk_vec + args.map.pad_vec) * 16;

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        LoaderPlan<kMaxInsts> lp;
        const int valid_blocks = args.contiguous ? at_eff : args.map.blocks;
        const int valid_vec = args.contiguous ? args.map.blk_vec : dt_eff / VW;
        make_loader_plan<kMaxInsts>(args.map, args.insts, VW, EB, args.n_in, valid_blocks, valid_vec,
                                    t - kConsumerThreads, &lp);
        auto issue = [&](int s) {
            const int64_t n0 = stage_row(s);
            const int64_t row_end = min(args.batch, n0 + R);
            issue_stage<kMaxInsts>(lp, args.insts, X + n0 * args.n_in + chunk_base,
                                   stage_limit(n0, row_end, args.n_in, EB), lds + (s % kStages) * kStageBytes);
        };
        for (int s = 0; s < kStages - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // stage s has landed once only the stages issued after it remain
            wait_vmcnt_upto(min(kStages - 2, nsteps - 1 - s) * args.insts);
            lds_barrier();
            if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    int g, al_l, de_l;   // beta group, alpha within the tile, first delta within the tile
    if (LANE && ILV) {
        // lanes ordered (alpha, beta, delta run): for each beta the lanes of
        // one alpha store its d outputs next to those of the next beta
        const int runs = args.dt / DV;              // delta runs per alpha
        const int run = t % runs;
        g = (t / runs) % G;
        al_l = t / (runs * G);
        de_l = run * DV;
    } else if (LANE) {
        g = t / P;
        const int p = t - g * P;
        const int runs = args.dt / DV;              // delta runs per alpha
        al_l = p / runs;
        de_l = (p - al_l * runs) * DV;
    } else {
        g = t % G;
        al_l = t / G;
        de_l = 0;
    }
    const int alpha = alpha0 + al_l;
    const int delta = delta0 + de_l;
    const bool active = al_l < at_eff && (LANE ? (de_l < dt_eff) : true);

    // weights: kr[j][dv][gamma] = K[alpha][delta + dv][g*NB + j][gamma]
    float kr[NB][DV][C];
#pragma unroll
    for (int dv = 0; dv < DV; ++dv)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const TW* kp = K + ((int64_t(alpha) * d + delta + dv) * B + g * NB + j) * C;
#pragma unroll
            for (int gm = 0; gm < C; ++gm) kr[j][dv][gm] = active ? to_f32(kp[gm]) : 0.0f;
        }

    // LDS offset of this thread's X within a staged row, and the gamma stride.
    const int xl_off = !active ? 0
                     : LANE ? (args.contiguous ? al_l * pitch_bytes + de_l * EB : de_l * EB)
                            : al_l * pitch_bytes;
    const int gstride = LANE ? (args.contiguous ? d : args.dt) * EB : 0;
    const int64_t yoff = LANE ? (int64_t(alpha) * B + g * NB) * d + delta
                              : (int64_t(alpha) * B + g * NB) * DV;

    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();
        const unsigned char* base = lds + (s % kStages) * kStageBytes;
        const int64_t n0 = stage_row(s);
        const int rows = static_cast<int>(min(int64_t(R), args.batch - n0));
#pragma unroll 1
        for (int r = 0; r < rows; ++r) {
            const unsigned char* xr = base + r * row_bytes + xl_off;
            float acc[NB][DV];
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int dv = 0; dv < DV; ++dv) acc[j][dv] = 0.0f;
            if (LANE) {
#pragma unroll
                for (int gm = 0; gm < C; ++gm) {
                    float x[DV];
                    const unsigned char* xp = xr + gm * gstride;
                    if constexpr (DV == 4 && EB == 4) {
                        const floatx4 w = *reinterpret_cast<const floatx4*>(xp);
                        x[0] = w[0]; x[1] = w[1]; x[2] = w[2]; x[3] = w[3];
                    } else if constexpr (DV == 4) {
                        const u32x2 w = *reinterpret_cast<const u32x2*>(xp);
                        x[0] = bf16_lo(w[0]); x[1] = bf16_hi(w[0]); x[2] = bf16_lo(w[1]); x[3] = bf16_hi(w[1]);
                    } else {
                        x[0] = to_f32(*reinterpret_cast<const TX*>(xp));
                    }
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int dv = 0; dv < DV; ++dv) acc[j][dv] = fmaf(kr[j][dv][gm], x[dv], acc[j][dv]);
                }
            } else {
                // the slab holds c*DV elements, element e = gamma*DV + delta
#pragma unroll
                for (int v = 0; v < C * DV / VW; ++v) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(xr + v * 16);
                    float xv[VW];
                    if constexpr (EB == 4) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) xv[e] = __uint_as_float(w[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) { xv[2 * e] = bf16_lo(w[e]); xv[2 * e + 1] = bf16_hi(w[e]); }
                    }
#pragma unroll
                    for (int e = 0; e < VW; ++e) {
                        const int el = v * VW + e;
                        const int gm = el / DV;
                        const int dv = el - gm * DV;
#pragma unroll
                        for (int j = 0; j < NB; ++j) acc[j][dv] = fmaf(kr[j][dv][gm], xv[e], acc[j][dv]);
                    }
                }
            }
            if (active) {
                float* yrow = Y + (n0 + r) * args.n_out + yoff;
                if (LANE) {
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        if constexpr (DV == 4)
                            __builtin_nontemporal_store(floatx4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]},
                                                        reinterpret_cast<floatx4*>(yrow + int64_t(j) * d));
                        else
                            __builtin_nontemporal_store(acc[j][0], yrow + int64_t(j) * d);
                    }
                } else {
                    constexpr int NOUT = NB * DV;
                    if constexpr (NOUT % 4 == 0) {
#pragma unroll
                        for (int v = 0; v < NOUT / 4; ++v)
                            __builtin_nontemporal_store(
                                floatx4{acc[(4 * v + 0) / DV][(4 * v + 0) % DV], acc[(4 * v + 1) / DV][(4 * v + 1) % DV],
                                        acc[(4 * v + 2) / DV][(4 * v + 2) % DV], acc[(4 * v + 3) / DV][(4 * v + 3) % DV]},
                                reinterpret_cast<floatx4*>(yrow) + v);
                    } else {
#pragma unroll
                        for (int e = 0; e < NOUT; ++e) __builtin_nontemporal_store(acc[e / DV][e % DV], yrow + e);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: tile geometry and dispatch.

struct ValuGeom {
    bool lane;
    bool ilv;   // lane mode with lanes ordered (alpha, beta, delta run), one beta each
    int dv, nb, g, p, at, dt, tiles_delta, n_tiles, contiguous, vw, insts, stages;
    StageMap map;
};

// The largest tile width <= cap that splits n into equal tiles (as equal as
// the tile count allows), so no tile is left nearly empty.
int balanced(int n, int cap) {
    if (cap < 1) return 0;
    const int tiles = (n + cap - 1) / cap;
    return (n + tiles - 1) / tiles;
}

bool geom_for(const Shape& s, int xt, ValuGeom* gm) {
    const int eb = elem_bytes(xt);
    const int vw = 16 / eb;
    const int b = s.b, c = s.c, d = s.d;
    if (!((b == 4 || b == 8 || b == 16) && (c == 4 || c == 8 || c == 16))) return false;
    gm->vw = vw;
    StageMap& m = gm->map;
    if (d >= 8) {
        if (d % vw != 0) return false;
        gm->lane = true;
        gm->dv = (d % 4 == 0) ? 4 : 1;
        // d <= 32: an alpha's outputs for one beta are at most 128 bytes, so
        // with beta-major lanes a store instruction writes pieces of lines
        // (the other betas' stores fill them later); one beta per thread with
        // lanes ordered (alpha, beta, run) stores whole lines. Measured
        // (16,384 rows): (128, 4, 4, 8) 2.8 -> 4.4 TB/s, (64, 8, 8, 8)
        // 3.1 -> 3.9; (64, 4, 4, 16) 119 -> 107 us, (32, 8, 8, 16) 125 -> 108,
        // (16, 8, 8, 32) 122 -> 108; (32, 4, 4, 32) unchanged
        gm->ilv = gm->dv == 4 && d / gm->dv <= 8;
        gm->nb = gm->ilv ? 1 : nb_rule(b, c, gm->dv);
        gm->g = b / gm->nb;
        gm->p = kConsumerThreads / gm->g;
        const int span = gm->p * gm->dv;            // deltas one group covers
        if (d >= span) {
            gm->dt = span;
            gm->at = 1;
            gm->contiguous = 0;
            m.blocks = c;
            m.blk_vec = span / vw;
            m.pad_vec = 0;
            m.gstride = d;
            m.row_vec = c * m.blk_vec;
        } else {
            gm->dt = d;
            gm->contiguous = 1;
            m.blk_vec = c * d / vw;
            // alpha-slab pitch congruent to d elements modulo 256 bytes, so
            // lanes reading consecutive (alpha, delta) hit consecutive banks
            const int slab = c * d * eb;
            const int want = (d * eb) % 256;
            const int pad = ((want - slab) % 256 + 256) % 256;
            if (pad % 16 != 0) return false;
            m.pad_vec = pad / 16;
            // as many alphas as the threads cover and one stage row holds
            gm->at = balanced(s.a, std::min(span / d, kMaxInsts * 64 / (m.blk_vec + m.pad_vec)));
            if (gm->at < 1) return false;
            m.blocks = gm->at;
            m.gstride = c * d;
            m.row_vec = gm->at * (m.blk_vec + m.pad_vec);
        }
    } else {
        if (d != 1 && d != 2 && d != 4) return false;
        if ((c * d) % vw != 0) return false;
        gm->lane = false;
        gm->ilv = false;
        gm->dv = d;
        gm->nb = nb_pick(b, c, d, false);
        gm->g = b / gm->nb;
        gm->p = kConsumerThreads / gm->g;
        gm->dt = d;
        gm->contiguous = 1;
        m.blk_vec = c * d / vw;
        const int slab = c * d * eb;
        // odd multiple of 16 bytes: 16 consecutive alpha slabs start in
        // distinct 16-byte bank groups
        m.pad_vec = (slab % 32 == 0) ? 1 : 0;
        gm->at = balanced(s.a, std::min(gm->p, kMaxInsts * 64 / (m.blk_vec + m.pad_vec)));
        if (gm->at < 1) return false;
        m.blocks = gm->at;
        m.gstride = c * d;
        m.row_vec = gm->at * (m.blk_vec + m.pad_vec);
    }
    if (m.row_vec > kMaxInsts * 64) return false;
    m.rows = std::max(1, std::min(16, kTargetVec / m.row_vec));
    // the loader addresses a stage with 32-bit byte offsets
    while (m.rows > 1 && int64_t(m.rows) * s.n_in * eb >= (int64_t(1) << 31)) --m.rows;
    if (int64_t(m.rows) * s.n_in * eb >= (int64_t(1) << 31)) return false;
    gm->insts = (m.rows * m.row_vec + 63) / 64;
    // ring depth: as many stages as fit the per-workgroup LDS budget, 3..8,
    // with the loader's wait count (stages - 2) * insts within vmcnt's range
    gm->stages = std::max(3, std::min(8, kLdsPerGroup / (gm->insts * 1024)));
    while (gm->stages > 3 && (gm->stages - 2) * gm->insts > 63) --gm->stages;
    if ((gm->stages - 2) * gm->insts > 63) return false;
    const int64_t tiles_alpha = (s.a + gm->at - 1) / gm->at;
    gm->tiles_delta = gm->contiguous ? 1 : (d + gm->dt - 1) / gm->dt;
    const int64_t nt = tiles_alpha * gm->tiles_delta;
    if (nt > (int64_t(1) << 30)) return false;
    gm->n_tiles = static_cast<int>(nt);
    return true;
}

// Rows per workgroup: a multiple of the stage rows, chosen so that the grid
// is about one wave of workgroups with equal shares, unless the tiles alone
// already fill it. With X stages of 16 KB or more one workgroup per compute
// unit streams faster than two (measured on the b, c = 4 and 8 square
// patterns: about 5.0 against 4.3 TB/s); with smaller stages two do.
int64_t rows_per_split(const ValuGeom& gm, int64_t batch, int num_cus, int rows_per_block) {
    const int R = gm.map.rows;
    const int64_t steps_total = (batch + R - 1) / R;
    int64_t steps;
    if (rows_per_block > 0) {
        steps = std::max<int64_t>(1, (rows_per_block + R - 1) / R);
    } else {
        const int per_cu = gm.insts >= 16 ? 1 : 2;
        const int64_t resident = int64_t(std::max(num_cus, 1)) * per_cu;
        const int64_t splits = std::max<int64_t>(1, resident / std::max(gm.n_tiles, 1));
        steps = (steps_total + splits - 1) / splits;
        // Stages of three rows (16 alpha slabs of 4 KB or 64 of 1 KB per
        // row): two rounds of half-size workgroups ran faster than one round
        // (measured with forced rows per workgroup: (64, 8, 8, 8) 132 -> 109
        // us, (256, 4, 4, 4) 132 -> 107 us at 16,384 rows, 43 steps per
        // workgroup); with a dozen steps per workgroup (4,096 rows) and for
        // other stage shapes it did not gain or lost.
        if (R == 3 && steps >= 32) steps = (steps + 1) / 2;
    }
    steps = std::max<int64_t>(1, std::min(steps, steps_total));
    return steps * R;
}

template <typename TX, typename TW, int B, int C>
ks_status_t launch_bc(const FactorCall& f, const ValuGeom& gm, const ValuArgs& args, dim3 grid) {
    const size_t lds = size_t(gm.stages) * gm.insts * 1024;
    const TX* X = static_cast<const TX*>(f.X);
    const TW* K = static_cast<const TW*>(f.W);
    const dim3 block(kStreamThreads);
    if (gm.lane && gm.dv == 4) {
        if (gm.ilv)
            return launch_kernel(valu_kernel<TX, TW, B, C, 4, true, true>, grid, block, lds, f.stream, X, K, f.Y,
                                 args);
        return launch_kernel(valu_kernel<TX, TW, B, C, 4, true, false>, grid, block, lds, f.stream, X, K, f.Y, args);
    } else if (gm.lane) {
        return launch_kernel(valu_kernel<TX, TW, B, C, 1, true, false>, grid, block, lds, f.stream, X, K, f.Y, args);
    } else if (f.s.d == 1) {
        return launch_kernel(valu_kernel<TX, TW, B, C, 1, false, false>, grid, block, lds, f.stream, X, K, f.Y, args);
    } else if (f.s.d == 2) {
        return launch_kernel(valu_kernel<TX, TW, B, C, 2, false, false>, grid, block, lds, f.stream, X, K, f.Y, args);
    } else {
        return launch_kernel(valu_kernel<TX, TW, B, C, 4, false, false>, grid, block, lds, f.stream, X, K, f.Y, args);
    }
}

template <typename TX, typename TW, int B>
ks_status_t launch_b(const FactorCall& f, const ValuGeom& gm, const ValuArgs& args, dim3 grid) {
    switch (f.s.c) {
        case 4: return launch_bc<TX, TW, B, 4>(f, gm, args, grid);
        case 8: return launch_bc<TX, TW, B, 8>(f, gm, args, grid);
        case 16: return launch_bc<TX, TW, B, 16>(f, gm, args, grid);
    }
    return KS_ERR_UNSUPPORTED;
}

template <typename TX, typename TW>
ks_status_t launch_types(const FactorCall& f, const ValuGeom& gm, const ValuArgs& args, dim3 grid) {
    switch (f.s.b) {
        case 4: return launch_b<TX, TW, 4>(f, gm, args, grid);
        case 8: return launch_b<TX, TW, 8>(f, gm, args, grid);
        case 16: return launch_b<TX, TW, 16>(f, gm, args, grid);
    }
    return KS_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool valu_supports(const Shape& s, int xt, int wt) {
    (void)wt;
    ValuGeom gm;
    return geom_for(s, xt, &gm);
}

int valu_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len) {
    (void)wt;
    ValuGeom gm;
    if (!geom_for(s, xt, &gm)) return std::snprintf(buf, len, "valu: unsupported");
    const int64_t rps = rows_per_split(gm, batch, num_cus, 0);
    return std::snprintf(buf, len,
                         "valu %s dv=%d: nb=%d groups=%d alphas/tile=%d deltas/tile=%d tiles=%d "
                         "rows/stage=%d rows/wg=%lld wgs=%lld stages=%d x %d KB",
                         gm.lane ? (gm.ilv ? "lane-interleaved" : "lane") : "slab", gm.dv, gm.nb, gm.g, gm.at,
                         gm.dt, gm.n_tiles,
                         gm.map.rows, static_cast<long long>(rps),
                         static_cast<long long>(gm.n_tiles * ((batch + rps - 1) / std::max<int64_t>(rps, 1))),
                         gm.stages, gm.insts);
}

ks_status_t launch_valu(const FactorCall& f) {
    ValuGeom gm;
    if (!geom_for(f.s, f.xt, &gm)) return KS_ERR_UNSUPPORTED;
    if (!aligned16(f.X) || !aligned16(f.Y)) return KS_ERR_UNSUPPORTED;
    if ((f.s.n_in * elem_bytes(f.xt)) % 16 != 0 || (f.s.n_out * 4) % 16 != 0) return KS_ERR_UNSUPPORTED;
    const int64_t rps = rows_per_split(gm, f.batch, f.num_cus, f.rows_per_block);
    const int64_t splits = (f.batch + rps - 1) / rps;
    const int64_t blocks = int64_t(gm.n_tiles) * splits;
    if (blocks > 0x7fffffff || rps > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    ValuArgs args;
    args.a = f.s.a;
    args.d = f.s.d;
    args.n_in = f.s.n_in;
    args.n_out = f.s.n_out;
    args.batch = f.batch;
    args.at = gm.at;
    args.dt = gm.dt;
    args.tiles_delta = gm.tiles_delta;
    args.n_tiles = gm.n_tiles;
    args.rows_per_split = static_cast<int>(rps);
    args.contiguous = gm.contiguous;
    args.insts = gm.insts;
    args.stages = gm.stages;
    args.xcd_remap = gm.contiguous ? 0 : 1;
    args.map = gm.map;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (f.xt == kF32 && f.wt == kF32) return launch_types<float, float>(f, gm, args, grid);
    if (f.xt == kBF16 && f.wt == kBF16) return launch_types<bf16_t, bf16_t>(f, gm, args, grid);
    if (f.xt == kF32 && f.wt == kBF16) return launch_types<float, bf16_t>(f, gm, args, grid);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
