// ks_mfma.hip -- KS matmul on the matrix cores for blocks with b, c >= 16.
//
// Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
//                                    * X[n][alpha][gamma][delta]
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph). For a
// fixed (alpha, delta) pair this is a dense product of the rows' c-vectors
// with the b x c block K[alpha][delta]: M = rows, N = b, K = c. With b and c
// of 16 or more that product fills v_mfma_f32_16x16x4_f32 tiles exactly, so
// the contraction runs on the matrix cores and the vector ALUs only move
// data. Most such shapes stay bound by HBM traffic (about 6 flop per byte at
// b = 64, c = 16); b = c = 128 is bound by the fp32 matrix rate. The kernel
// moves X and Y once, in whole 16-byte vectors, with no permutation pass
// through global memory (the same page, third sentence: a fused,
// output-stationary kernel).
//
// Workgroup: a tile of (alpha, delta) pairs and of BT of the b outputs (all
// of them unless the block is split), over a range of rows in steps of 16.
// One loader wave streams X into an LDS ring (ks_stream.h). Four compute
// waves, WN along the N tiles times WP along the pairs:
//  * hold the B operands of their N tiles and pairs in VGPRs for the whole
//    kernel (at most VB registers);
//  * per step and pair, read A operands (16 rows x 4 gammas) from LDS,
//    accumulate c/4 MFMAs in fp32 and write the 16 x 16 results into a Y
//    tile in LDS laid out like the rows of Y.
// The Y tile goes out in 16-byte vectors that cover whole segments of Y,
// stored either by the compute waves after each step or by a storer wave
// that drains step s-1 from a second Y buffer while step s computes.
// Splitting b over several tiles (which read the same X, through the L2)
// keeps the B operands of several pairs in registers when b and c are large.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"
#include "ks_tile.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsPerGroupDefault = 80 * 1024;   // two workgroups per compute unit
constexpr int kStoreQ = 4;                // storer: row-chunk vectors per lane

constexpr int kRows = 16;                 // rows per step: one MFMA M tile

// Waves along the N tiles and along the pairs (WN x WP = 4 compute waves),
// and N tiles per wave, for a tile of bt outputs.
__host__ __device__ constexpr int mfma_wn(int bt) { return bt / 16 < 4 ? bt / 16 : 4; }
__host__ __device__ constexpr int mfma_wp(int bt) { return 4 / mfma_wn(bt); }
__host__ __device__ constexpr int mfma_ntw(int bt) { return bt / 16 / mfma_wn(bt); }

// Pairs per tile, WP times a power of two: a wave's B operands take
// (TP / WP) * NTW * c / 4 VGPRs, at most vb; an X stage (16 rows of TP * c
// elements of eb bytes) stays within 48 KB; and three X stages plus the fp32
// Y tile (16 rows of TP * bt) stay within 150 KB of LDS.
__host__ __device__ constexpr int mfma_tp(int bt, int c, int eb, int vb) {
    int pw = vb / (mfma_ntw(bt) * (c / 4));
    if (pw < 1) pw = 1;
    int tp = pw * mfma_wp(bt);
    while (tp > mfma_wp(bt) && (kRows * tp * c * eb > 48 * 1024 ||
                                3 * kRows * tp * c * eb + kRows * tp * bt * 4 > 150 * 1024))
        tp /= 2;
    return tp;
}

// Tile shape of one (bt, c, element size, B-operand budget) instantiation.
template <int BT, int C, int EB, int VB>
struct MfmaShape {
    static constexpr int WN = mfma_wn(BT);             // waves along N
    static constexpr int WP = mfma_wp(BT);             // waves along pairs
    static constexpr int NTW = mfma_ntw(BT);           // N tiles per wave
    static constexpr int KS = C / 4;                   // MFMA K steps
    static constexpr int TP = mfma_tp(BT, C, EB, VB);  // pairs per tile
    static constexpr int PW = TP / WP;                 // pairs per wave
    static_assert(PW * WP == TP && PW * NTW * KS <= (VB > NTW * KS ? VB : NTW * KS), "B operand budget");
};

// Loader instructions (KB) per X stage: 16 rows of at most TP * c elements,
// plus one pad vector per row.
__host__ __device__ constexpr int mfma_stage_insts(int bt, int c, int eb, int vb) {
    return (kRows * (mfma_tp(bt, c, eb, vb) * c * eb / 16 + 1) + 63) / 64;
}

struct MfmaArgs {
    int a, d;
    int64_t n_in, n_out, batch;
    int at, dt;
    int tiles_delta, n_tiles;
    int rows_per_split;      // a multiple of the stage rows
    int contiguous;
    int qy;                  // Y vectors in one row chunk of the tile
    int insts;               // loader instructions per stage (stage = insts KB of LDS)
    int stages;              // LDS ring depth
    int ytile_bytes;         // LDS bytes of one Y tile buffer
    int xcd_remap;           // 1: renumber workgroups so neighbouring tiles share an XCD
    int vec_a;               // 1: the tile's deltas per gamma come in runs of 4 (dt % 4 == 0)
    int bsplit;              // tiles per (alpha, delta) block: b = bsplit * BT
    int b;                   // outputs per block (the K block stride is b * c)
    StageMap xmap;           // LDS layout of an X stage
    RowChunk yc;             // LDS layout of the Y tile and its global stores
};

// The threads that store Y tiles (the storer waves, or the compute waves
// when there are none) and their share of a tile. A row chunk of qy vectors
// needs S = ceil(qy / 64) waves' worth of lanes. With W >= S waves, wave w
// takes the 64 vectors of slot w % S in rows g, g + G, ... (g = w / S,
// G = W / S); with fewer waves, every wave takes slots w, w + W, ... of every
// row. Vector offsets are the same in every row and step, so they are
// computed once.
struct StoreTeam {
    int g, G;                 // first row and row stride of this wave
    int nq;                   // slots of this wave (wave-uniform, <= kStoreQ)
    int gq[kStoreQ];          // per slot: element offset in the Y row chunk
    int lq[kStoreQ];          // per slot: byte offset in the LDS row
    bool ok[kStoreQ];         // per slot: this lane has a vector there
};

template <typename A>
__device__ __forceinline__ void make_store_team(const A& args, int tid, int nthreads, int at_eff, int dt_eff,
                                                StoreTeam* st) {
    const int W = nthreads / 64, w = tid >> 6, lane = tid & 63;
    const int S = (args.qy + 63) / 64;
    int first, stride;
    if (S <= W) {
        st->G = W / S;
        st->g = w / S;
        st->nq = st->g < st->G ? 1 : 0;
        first = 64 * (w % S) + lane;
        stride = 0;
    } else {
        st->G = 1;
        st->g = 0;
        st->nq = min(kStoreQ, (S - w + W - 1) / W);
        first = 64 * w + lane;
        stride = 64 * W;
    }
#pragma unroll
    for (int j = 0; j < kStoreQ; ++j) {
        const int q = first + stride * j;
        st->ok[j] = false;
        st->gq[j] = st->lq[j] = 0;
        if (j < st->nq && q < args.qy)
            chunk_vector(args.yc, q, 4, at_eff, dt_eff, &st->gq[j], &st->lq[j], &st->ok[j]);
    }
}

// Stores rows [0, rows) of a Y tile staged in LDS at ys (R rows) to the Y
// rows that start at yrow0 (the tile's chunk of its first row). Per slot,
// RB rows at a time: all their LDS reads first (no branch between
// them), then the 16-byte nontemporal stores, so the LDS latency is paid
// once per batch. Rows past `rows` are read (clamped into the buffer) but
// not stored.
template <int RB, typename A>
__device__ __forceinline__ void store_tile_rows(const A& args, const StoreTeam& st, const unsigned char* ys,
                                                float* yrow0, int rows, int R) {
    // row phase, stride and slot count are the same on every lane of a wave
    const int g = __builtin_amdgcn_readfirstlane(st.g);
    const int G = __builtin_amdgcn_readfirstlane(st.G);
    const int nq = __builtin_amdgcn_readfirstlane(st.nq);
    const int64_t rstride = int64_t(G) * args.n_out;        // elements between a wave's rows
    const int lstride = G * args.yc.lds_row;                 // LDS bytes between a wave's rows
#pragma unroll
    for (int j = 0; j < kStoreQ; ++j) {
        if (j >= nq) break;
        const unsigned char* yl = ys + st.lq[j] + g * args.yc.lds_row;
        float* yg = yrow0 + st.gq[j] + int64_t(g) * args.n_out;
        for (int r0 = g; r0 < rows; r0 += G * RB) {
            u32x4 v[RB];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                // rows past R (possible only in the last batch) re-read row R - 1
                const int lofs = r0 + rr * G < R ? rr * lstride : (R - 1 - r0) * args.yc.lds_row;
                v[rr] = *reinterpret_cast<const u32x4*>(yl + lofs);
            }
#pragma unroll
            for (int rr = 0; rr < RB; ++rr)
                if (st.ok[j] && r0 + rr * G < rows)
                    __builtin_nontemporal_store(v[rr], reinterpret_cast<u32x4*>(yg + rr * rstride));
            yl += RB * lstride;
            yg += RB * rstride;
        }
    }
}

// NS = 0: the four compute waves also store each Y tile, after an LDS
// barrier. NS > 0: NS storer waves store tile s-1 from one of two Y buffers
// while the compute waves run the MFMAs of step s into the other, so the
// stores drain during the contraction instead of after it.
// NL loader waves: with two, each issues every other instruction of every
// stage and waits for its own (more LDS-DMA issue per step; measured faster
// on the b = c = 128 patterns with d >= 4, slower on others, so the fitted
// planner table chooses it per pattern).
template <int NL>
constexpr int mfma_load_end() { return kConsumerThreads + 64 * NL; }

template <typename TX, typename TW, int BT, int C, int NS, int VB, int NL>
__global__ __launch_bounds__(mfma_load_end<NL>() + 64 * NS) void mfma_kernel(const TX* __restrict__ X,
                                                                        const TW* __restrict__ K,
                                                                        float* __restrict__ Y, MfmaArgs args) {
    constexpr int EB = int(sizeof(TX));
    using S = MfmaShape<BT, C, EB, VB>;
    constexpr int NTW = S::NTW, WN = S::WN, WP = S::WP, PW = S::PW, KS = S::KS, R = kRows;
    constexpr int VWX = 16 / EB;
    constexpr int kMaxInsts = mfma_stage_insts(BT, C, EB, VB);
    static_assert(kMaxInsts <= 63, "vmcnt is six bits");
    const int kStageBytes = args.insts * 1024;
    const int kStages = args.stages;

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* const ys0 = lds + kStages * kStageBytes;

    const int t = threadIdx.x;
    const int blk = args.xcd_remap ? xcd_logical_block(blockIdx.x, gridDim.x) : int(blockIdx.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    // tiles that read the same X (the b splits of one block) are neighbours
    const int tad = tile / args.bsplit;
    const int beta0 = (tile - tad * args.bsplit) * BT;
    const int ta = tad / args.tiles_delta;
    const int td = tad - ta * args.tiles_delta;
    const int alpha0 = ta * args.at;
    const int delta0 = td * args.dt;
    const int d = args.d;
    const int at_eff = min(args.at, args.a - alpha0);
    const int dt_eff = min(args.dt, d - delta0);
    const bool contig = args.contiguous != 0;
    const int64_t xg0 = int64_t(alpha0) * C * d + (contig ? 0 : delta0);
    const int64_t yg0 = (int64_t(alpha0) * args.b + beta0) * d + (contig ? 0 : delta0);

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + R - 1) / R);
    const int xrow_bytes = args.xmap.row_vec * 16;
    const int xblk_bytes = args.xmap.blk_vec * 16;   // no per-block padding in X stages

    if constexpr (NS > 0) {
        if (t >= mfma_load_end<NL>()) {
            // ---------------------------------------------------- storer waves
            // Issue priority over the compute waves on the same SIMD: their
            // MFMA bursts otherwise delay the stores (measured 4-9 % on the
            // ViT and b = c = 128 shapes).
            __builtin_amdgcn_s_setprio(3);
            StoreTeam team;
            make_store_team(args, t - mfma_load_end<NL>(), 64 * NS, at_eff, dt_eff, &team);
            auto store_tile = [&](int s) {
                const int64_t n0 = row_begin + int64_t(s) * R;
                store_tile_rows<8>(args, team, ys0 + (s & 1) * args.ytile_bytes, Y + n0 * args.n_out + yg0,
                                static_cast<int>(min(int64_t(R), row_end - n0)), R);
            };
            for (int s = 0; s < nsteps; ++s) {
                lds_barrier();                               // stage s ready
                if (s > 0) store_tile(s - 1);
                lds_barrier();                               // Y tile s written
            }
            store_tile(nsteps - 1);
            return;
        }
    }

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        LoaderPlan<kMaxInsts> lp;
        const int valid_blocks = contig ? at_eff : args.xmap.blocks;
        const int valid_vec = contig ? args.xmap.blk_vec : dt_eff / VWX;
        make_loader_plan<kMaxInsts>(args.xmap, args.insts, VWX, EB, args.n_in, valid_blocks, valid_vec,
                                    (t - kConsumerThreads) & 63, &lp);
        const int L = (t - kConsumerThreads) >> 6;                // loader wave
        const int own = (args.insts - L + NL - 1) / NL;          // its instructions per stage
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * R;
            if constexpr (NL == 1) {
                issue_stage<kMaxInsts>(lp, args.insts, X + n0 * args.n_in + xg0,
                                       stage_limit(n0, row_end, args.n_in, EB), lds + (s % kStages) * kStageBytes);
            } else {
                issue_stage_part<kMaxInsts>(lp, args.insts, X + n0 * args.n_in + xg0,
                                            stage_limit(n0, row_end, args.n_in, EB),
                                            lds + (s % kStages) * kStageBytes, L, NL);
            }
        };
        for (int s = 0; s < kStages - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // stage s has landed once only the stages issued after it remain
            wait_vmcnt_upto(min(63, min(kStages - 2, nsteps - 1 - s) * own));
            lds_barrier();                                   // stage s ready
            if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
            lds_barrier();                                   // Y tile written
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int wave = t >> 6;
    const int lane = t & 63;
    const int wn = wave % WN;                     // N tiles wn * NTW ..
    const int wp = wave / WN;                     // pairs wp, wp + WP, ..

    const int gsx = contig ? d * EB : xblk_bytes;          // X: gamma stride in LDS
    // A operands of 4 pairs with consecutive deltas (same alpha) lie side by
    // side in the X stage, so one 4-element LDS read feeds all four. Single
    // reads of one pair's operands (16 rows x 4 gammas) fall on a quarter of
    // the banks when the gamma stride is a multiple of 16 bytes: 8-way
    // conflicts, which the vector reads avoid and with a quarter of the LDS
    // instructions. Used for the large contractions, where a wave holds 4
    // pairs or more.
    constexpr int VDX = (C >= 64 && PW % 4 == 0) ? 4 : 1;
    const bool vec = VDX > 1 && args.vec_a != 0;
    const int bsy = contig ? d * 4 : args.yc.seg_lds;      // Y: beta stride in LDS
    int xoff[PW], yoff[PW];
    bool pv[PW];
    float breg[PW][NTW][KS];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int p = vec ? 4 * (wp + WP * (i / 4)) + (i % 4) : wp + WP * i;   // runs of 4 deltas
        const int al = p / args.dt;
        const int de = p - al * args.dt;
        pv[i] = p < args.at * args.dt && al < at_eff && de < dt_eff;
        xoff[i] = contig ? al * xblk_bytes + de * EB : de * EB;
        yoff[i] = contig ? al * args.yc.lds_slab + de * 4 : de * 4;
        const TW* kp = K + ((int64_t(alpha0 + al) * d + delta0 + de) * args.b + beta0) * C;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int beta = (wn * NTW + nt) * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int gamma = ks * 4 + (lane >> 4);
                breg[i][nt][ks] = pv[i] ? to_f32(kp[beta * C + gamma]) : 0.0f;
            }
        }
    }

    StoreTeam team;
    if constexpr (NS == 0) make_store_team(args, t, kConsumerThreads, at_eff, dt_eff, &team);

    const int arow = lane & 15;                   // A operand row of this lane
    const int akk = lane >> 4;                    // A operand k (gamma within a step)
    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();                                                   // stage s ready
        const unsigned char* xcur = lds + (s % kStages) * kStageBytes;
        unsigned char* const ys = NS > 0 ? ys0 + (s & 1) * args.ytile_bytes : ys0;
        if (VDX > 1 && vec) {
#pragma unroll
            for (int j = 0; j < PW / VDX; ++j) {
                if (!pv[VDX * j]) continue;
                floatx4 acc[VDX][NTW];
#pragma unroll
                for (int u = 0; u < VDX; ++u)
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) acc[u][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                const unsigned char* xa = xcur + arow * xrow_bytes + xoff[VDX * j] + akk * gsx;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    float av[4];
                    load4_f32(reinterpret_cast<const TX*>(xa + ks * 4 * gsx), av);
#pragma unroll
                    for (int u = 0; u < VDX; ++u)
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt)
                            acc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], breg[VDX * j + u][nt][ks],
                                                                              acc[u][nt], 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < VDX; ++u) {
                    if (!pv[VDX * j + u]) continue;
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) {
                        const int beta = (wn * NTW + nt) * 16 + (lane & 15);
                        unsigned char* yb = ys + yoff[VDX * j + u] + beta * bsy;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = 4 * (lane >> 4) + v;
                            *reinterpret_cast<float*>(yb + row * args.yc.lds_row) = acc[u][nt][v];
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < PW; ++i) {
                if (!pv[i]) continue;
                floatx4 acc[NTW];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                const unsigned char* xa = xcur + arow * xrow_bytes + xoff[i] + akk * gsx;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const float av = to_f32(*reinterpret_cast<const TX*>(xa + ks * 4 * gsx));
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, breg[i][nt][ks], acc[nt], 0, 0, 0);
                }
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const int beta = (wn * NTW + nt) * 16 + (lane & 15);
                    unsigned char* yb = ys + yoff[i] + beta * bsy;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = 4 * (lane >> 4) + v;
                        *reinterpret_cast<float*>(yb + row * args.yc.lds_row) = acc[nt][v];
                    }
                }
            }
        }
        lds_barrier();                                                   // Y tile written
        if constexpr (NS == 0) {
            const int64_t n0 = row_begin + int64_t(s) * R;
            store_tile_rows<4>(args, team, ys, Y + n0 * args.n_out + yg0, static_cast<int>(min(int64_t(R), row_end - n0)),
                            R);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

struct MfmaGeom {
    int tp, r, at, dt, tiles_delta, n_tiles, contiguous, qy, insts, stages;
    int ns;        // storer waves (0: the compute waves store)
    int ytile;     // LDS bytes of one Y buffer
    int vb;        // B-operand VGPR budget of the instantiation (64 or 128)
    int bsplit;    // tiles per (alpha, delta) block along b
    int bt;        // outputs per tile (b / bsplit)
    StageMap xmap;
    RowChunk yc;
    size_t lds;
};

// Workgroups of this kernel that one compute unit holds: its LDS (160 KB)
// and its wave slots (with the 64-register B budget the kernel takes
// 110-140 VGPRs, 3-4 waves per SIMD, or 80-90 with a storer wave, 5 per
// SIMD; with the 128-register budget 150-190 VGPRs, 2-3 per SIMD).
int mfma_groups_per_cu(size_t lds, int ns, int vb) {
    const size_t waves = vb > 64 ? (ns ? 12 : 8) : (ns ? 20 : 12);
    return static_cast<int>(std::min<size_t>((160 * 1024) / std::max<size_t>(lds, 1), waves / (5 + ns)));
}

bool pow2_block(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }

// The 128-register B budget is built for tiles whose c is 64 or 128, the
// 32-register one for tiles of 16 or 32 outputs.
bool vb_built(int bt, int c, int vb) {
    return vb == 64 || (vb == 128 && bt >= 32 && c >= 64) || (vb == 32 && bt <= 32);
}

// Smallest pad (in 16-byte vectors) making a row pitch of `vec` vectors an
// odd multiple of 16 bytes modulo 256, so 16 consecutive rows start in
// distinct 16-byte bank groups.
int row_pad(int vec) {
    int pad = 0;
    while (((vec + pad) % 16) % 2 == 0) ++pad;
    return pad;
}

// Geometry of one candidate (B budget vb, b split into bsplit tiles).
bool geom_for(const Shape& s, int xt, int vb, int bsplit, int store_waves, MfmaGeom* g) {
    const int b = s.b, c = s.c, d = s.d;
    if (b % bsplit != 0) return false;
    const int bt = b / bsplit;
    if (!pow2_block(bt) || !pow2_block(c) || !vb_built(bt, c, vb)) return false;
    const int eb = elem_bytes(xt);
    const int vwx = 16 / eb;
    // LDS budget per workgroup. 80 KB keeps two workgroups on a compute
    // unit. Tiles of 16 or 32 outputs with d < 16 ran faster as one
    // workgroup per unit with 86 KB (two X alpha slabs per stage and a
    // storer wave: 5.3-5.9 against 4.3-5.4 TB/s on the b = c = 16, 32 square
    // patterns and the last butterfly factor); with d >= 16 they did not.
    const int kLdsPerGroup = (bt <= 32 && d < 16) ? 86 * 1024 : kLdsPerGroupDefault;
    g->vb = vb;
    g->bsplit = bsplit;
    g->bt = bt;
    g->tp = mfma_tp(bt, c, eb, vb);
    g->r = kRows;
    const int kStageInsts = mfma_stage_insts(bt, c, eb, vb);
    if (kStageInsts > 63) return false;
    // the loader addresses a stage with 32-bit byte offsets
    if (int64_t(g->r) * s.n_in * eb >= (int64_t(1) << 31)) return false;
    StageMap& xm = g->xmap;
    RowChunk& yc = g->yc;
    xm.rows = g->r;
    xm.pad_vec = 0;
    if (d <= g->tp) {
        if ((c * d) % vwx != 0) return false;
        // as many alphas as the pairs allow, while the X stage fits and the
        // whole workgroup stays within about 80 KB of LDS (two per CU), with
        // two Y buffers (a storer wave) if possible, else with one
        const int blk = c * d / vwx;
        auto fits = [&](int at, int ybufs) {
            const int xv = at * blk;
            const int insts = (g->r * (xv + row_pad(xv)) + 63) / 64;
            const size_t lds = size_t(3) * insts * 1024 + size_t(ybufs) * g->r * (size_t(at) * bt * d * 4 + 16);
            return g->r * (xv + row_pad(xv)) <= kStageInsts * 64 && lds <= kLdsPerGroup;
        };
        const int at_max = std::max(1, g->tp / d);
        g->at = 0;
        for (int ybufs = 2; ybufs >= 1 && g->at == 0; --ybufs)
            for (int at = at_max; at >= 1 && g->at == 0; --at)
                if (fits(at, ybufs)) g->at = at;
        if (g->at == 0) g->at = 1;
        // a power of two, so that alpha tiles split a (a power of two in
        // the butterfly and square families) evenly: (4096, 16, 16, 1) ran
        // 274 tiles of 15 alphas at 3.8 TB/s, 512 tiles of 8 at 5.3 TB/s
        while (g->at & (g->at - 1)) g->at &= g->at - 1;
        g->dt = d;
        g->contiguous = 1;
        xm.blocks = g->at;
        xm.blk_vec = blk;
        xm.gstride = c * d;
        xm.row_vec = g->at * xm.blk_vec;
        yc.contiguous = 1;
        yc.slab = bt * d;
        yc.slab_global = b * d;
        yc.lds_slab = bt * d * 4;
        yc.lds_row = g->at * yc.lds_slab + 16;
        yc.nseg = yc.seg_global = yc.seg_lds = yc.seg_cap = 0;
    } else {
        // one alpha, tp deltas: segments of tp elements, d apart
        if (g->tp % vwx != 0 || d % vwx != 0 || g->tp % 4 != 0 || d % 4 != 0) return false;
        g->at = 1;
        g->dt = g->tp;
        g->contiguous = 0;
        xm.blocks = c;
        xm.blk_vec = g->tp / vwx;
        xm.gstride = d;
        xm.row_vec = c * xm.blk_vec;
        yc.contiguous = 0;
        yc.slab = yc.slab_global = yc.lds_slab = 0;
        yc.nseg = bt;
        yc.seg_global = d;
        yc.seg_cap = g->tp;
        yc.seg_lds = g->tp * 4;
        yc.lds_row = bt * g->tp * 4 + 16;
    }
    xm.row_vec += row_pad(xm.row_vec);
    if (xm.rows * xm.row_vec > kStageInsts * 64) return false;
    const int64_t tiles_alpha = (s.a + g->at - 1) / g->at;
    g->tiles_delta = g->contiguous ? 1 : (d + g->dt - 1) / g->dt;
    const int64_t nt_all = tiles_alpha * g->tiles_delta * bsplit;
    if (nt_all > (int64_t(1) << 30)) return false;
    g->n_tiles = static_cast<int>(nt_all);
    g->qy = g->contiguous ? g->at * bt * d / 4 : bt * g->dt / 4;
    g->insts = (xm.rows * xm.row_vec + 63) / 64;
    if (g->insts > 63) return false;
    // ring depth: as many stages as fit next to the Y buffers in the
    // per-workgroup LDS budget, 3..8, with the loader's wait count
    // (stages - 2) * insts within vmcnt's range
    const int64_t ytile = int64_t(g->r) * yc.lds_row;
    auto ring = [&](int64_t ybytes) {
        int st = static_cast<int>(
            std::max<int64_t>(3, std::min<int64_t>(8, (kLdsPerGroup - ybytes) / (g->insts * 1024))));
        while (st > 3 && (st - 2) * g->insts > 63) --st;
        return st;
    };
    const int st0 = ring(ytile), st1 = ring(2 * ytile);
    const size_t lds0 = size_t(st0) * g->insts * 1024 + size_t(ytile);
    const size_t lds1 = size_t(st1) * g->insts * 1024 + size_t(2 * ytile);
    // A storer wave with a second Y buffer lets the stores of one step drain
    // during the next step's MFMAs; take it unless its LDS or its extra wave
    // costs a workgroup per compute unit.
    if (g->qy > 64 * 4 * kStoreQ) return false;   // the compute waves' store team covers a row chunk
    const bool storer_fits = g->qy <= 64 * kStoreQ && lds1 <= 160 * 1024;
    if (store_waves == KS_STORE_DEDICATED && !storer_fits) return false;
    const bool storer = store_waves == KS_STORE_DEDICATED ||
                        (store_waves == KS_STORE_AUTO && storer_fits &&
                         mfma_groups_per_cu(lds1, 1, vb) >= mfma_groups_per_cu(lds0, 0, vb));
    if (storer) {
        g->ns = 1;
        g->stages = st1;
        g->lds = lds1;
    } else {
        g->ns = 0;
        g->stages = st0;
        g->lds = lds0;
    }
    if ((g->stages - 2) * g->insts > 63) return false;
    g->ytile = static_cast<int>(ytile);
    return g->lds <= 160 * 1024;
}

// The planner's tile: the first candidate whose X runs (the contiguous
// part of a row that one tile reads) are at least 32 bytes, else the first
// that runs at all. Candidates go from the cheapest (32 or 64 B registers
// per wave, whole blocks) to wider register budgets and split blocks.
// tile: 0 = the first candidate that reads X in runs of >= 32 bytes (or a
// contiguous tile), else the first that fits; 1..KS_MFMA_TILES = that
// candidate only.
bool choose_geom(const Shape& s, int xt, int store_waves, int tile, MfmaGeom* g) {
    static const int kCand[][2] = {{32, 1}, {64, 1}, {128, 1}, {128, 2}, {64, 2}, {128, 4}, {64, 4}};
    static_assert(sizeof(kCand) / sizeof(kCand[0]) == KS_MFMA_TILES, "tile candidates");
    if (tile < 0 || tile > KS_MFMA_TILES) return false;
    if (tile > 0) return geom_for(s, xt, kCand[tile - 1][0], kCand[tile - 1][1], store_waves, g);
    const int eb = elem_bytes(xt);
    bool found = false;
    for (const auto& cand : kCand) {
        MfmaGeom t;
        if (!geom_for(s, xt, cand[0], cand[1], store_waves, &t)) continue;
        // The 32-register budget halves the pairs per tile: only for
        // contiguous tiles (segmented ones would read half-length runs).
        // There it measured 5.6-5.9 against 5.1-5.4 TB/s on the b = c = 32
        // square patterns with d <= 8.
        if (cand[0] == 32 && !t.contiguous) continue;
        if (t.contiguous || t.dt * eb >= 32) {
            *g = t;
            return true;
        }
        if (!found) {
            *g = t;
            found = true;
        }
    }
    return found;
}

// Rows per workgroup: a multiple of the stage rows, so that the grid is about
// one resident wave of workgroups with equal shares.
int64_t rows_per_split(const MfmaGeom& g, int64_t batch, int num_cus, int rows_per_block) {
    const int64_t steps_total = (batch + g.r - 1) / g.r;
    int64_t steps;
    if (rows_per_block > 0) {
        steps = std::max<int64_t>(1, (rows_per_block + g.r - 1) / g.r);
    } else {
        const int64_t per_cu = std::max(1, mfma_groups_per_cu(g.lds, g.ns, g.vb));
        const int64_t resident = int64_t(std::max(num_cus, 1)) * per_cu;
        const int64_t splits = std::max<int64_t>(1, resident / std::max(g.n_tiles, 1));
        steps = (steps_total + splits - 1) / splits;
    }
    steps = std::max<int64_t>(1, std::min(steps, steps_total));
    return steps * g.r;
}

template <typename TX, typename TW, int BT, int C, int VB, int NL>
ks_status_t launch_nl(const FactorCall& f, const MfmaGeom& g, const MfmaArgs& args, dim3 grid) {
    constexpr int end = mfma_load_end<NL>();
    if (g.ns == 1)
        return launch_kernel(mfma_kernel<TX, TW, BT, C, 1, VB, NL>, grid, dim3(end + 64), g.lds, f.stream,
                             static_cast<const TX*>(f.X), static_cast<const TW*>(f.W), f.Y, args);
    return launch_kernel(mfma_kernel<TX, TW, BT, C, 0, VB, NL>, grid, dim3(end), g.lds, f.stream,
                         static_cast<const TX*>(f.X), static_cast<const TW*>(f.W), f.Y, args);
}

template <typename TX, typename TW, int BT, int C, int VB>
ks_status_t launch_vb(const FactorCall& f, const MfmaGeom& g, const MfmaArgs& args, dim3 grid) {
    if constexpr (mfma_stage_insts(BT, C, int(sizeof(TX)), VB) <= 63) {
        // two loader waves only for the large blocks, where they can pay
        if constexpr (C >= 64) {
            if (f.mfma_loaders == 2) return launch_nl<TX, TW, BT, C, VB, 2>(f, g, args, grid);
        }
        if (f.mfma_loaders > 1) return KS_ERR_UNSUPPORTED;
        return launch_nl<TX, TW, BT, C, VB, 1>(f, g, args, grid);
    } else {
        return KS_ERR_UNSUPPORTED;
    }
}

template <typename TX, typename TW, int BT, int C>
ks_status_t launch_bc(const FactorCall& f, const MfmaGeom& g, const MfmaArgs& args, dim3 grid) {
    if (g.vb == 64) return launch_vb<TX, TW, BT, C, 64>(f, g, args, grid);
    if constexpr (BT <= 32) {
        if (g.vb == 32) return launch_vb<TX, TW, BT, C, 32>(f, g, args, grid);
    }
    if constexpr (BT >= 32 && C >= 64) {
        if (g.vb == 128) return launch_vb<TX, TW, BT, C, 128>(f, g, args, grid);
    }
    return KS_ERR_UNSUPPORTED;
}

template <typename TX, typename TW, int BT>
ks_status_t launch_b(const FactorCall& f, const MfmaGeom& g, const MfmaArgs& args, dim3 grid) {
    switch (f.s.c) {
        case 16: return launch_bc<TX, TW, BT, 16>(f, g, args, grid);
        case 32: return launch_bc<TX, TW, BT, 32>(f, g, args, grid);
        case 64: return launch_bc<TX, TW, BT, 64>(f, g, args, grid);
        case 128: return launch_bc<TX, TW, BT, 128>(f, g, args, grid);
    }
    return KS_ERR_UNSUPPORTED;
}

template <typename TX, typename TW>
ks_status_t launch_types(const FactorCall& f, const MfmaGeom& g, const MfmaArgs& args, dim3 grid) {
    switch (g.bt) {
        case 16: return launch_b<TX, TW, 16>(f, g, args, grid);
        case 32: return launch_b<TX, TW, 32>(f, g, args, grid);
        case 64: return launch_b<TX, TW, 64>(f, g, args, grid);
        case 128: return launch_b<TX, TW, 128>(f, g, args, grid);
    }
    return KS_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool mfma_supports(const Shape& s, int xt, int wt) {
    (void)wt;
    MfmaGeom g;
    return choose_geom(s, xt, KS_STORE_AUTO, 0, &g);
}

bool mfma_lds_supports(const Shape& s, int xt, int wt) { return mfma_supports(s, xt, wt); }

int mfma_describe(const Shape& s, int xt, int wt, int64_t batch, int num_cus, char* buf, size_t len,
                  int store_waves, int mfma_tile, int mfma_loaders) {
    (void)wt;
    MfmaGeom g;
    if (!choose_geom(s, xt, store_waves, mfma_tile, &g) && !choose_geom(s, xt, KS_STORE_AUTO, 0, &g))
        return std::snprintf(buf, len, "mfma: unsupported");
    const int64_t rps = rows_per_split(g, batch, num_cus, 0);
    return std::snprintf(buf, len,
                         "mfma 16x16x4f32: pairs/tile=%d (alphas=%d deltas=%d %s) outputs/tile=%d of %d "
                         "B regs=%d rows/wg=%lld wgs=%lld stages=%d x %d KB storers=%d loaders=%d lds=%zu",
                         g.tp, g.at, g.dt, g.contiguous ? "contiguous" : "segmented", g.bt, s.b, g.vb,
                         static_cast<long long>(rps),
                         static_cast<long long>(g.n_tiles * ((batch + rps - 1) / std::max<int64_t>(rps, 1))),
                         g.stages, g.insts, g.ns, (mfma_loaders == 2 && s.c >= 64) ? 2 : 1, g.lds);
}

ks_status_t launch_mfma(const FactorCall& f) { return launch_mfma_lds(f); }

ks_status_t launch_mfma_lds(const FactorCall& f) {
    MfmaGeom g;
    if (!choose_geom(f.s, f.xt, f.store_waves, f.mfma_tile, &g)) return KS_ERR_UNSUPPORTED;
    if (!aligned16(f.X) || !aligned16(f.Y)) return KS_ERR_UNSUPPORTED;
    if ((f.s.n_in * elem_bytes(f.xt)) % 16 != 0 || (f.s.n_out * 4) % 16 != 0) return KS_ERR_UNSUPPORTED;
    const int64_t rps = rows_per_split(g, f.batch, f.num_cus, f.rows_per_block);
    const int64_t splits = (f.batch + rps - 1) / rps;
    const int64_t blocks = int64_t(g.n_tiles) * splits;
    if (blocks > 0x7fffffff || rps > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    MfmaArgs args;
    args.a = f.s.a;
    args.d = f.s.d;
    args.n_in = f.s.n_in;
    args.n_out = f.s.n_out;
    args.batch = f.batch;
    args.at = g.at;
    args.dt = g.dt;
    args.tiles_delta = g.tiles_delta;
    args.n_tiles = g.n_tiles;
    args.rows_per_split = static_cast<int>(rps);
    args.contiguous = g.contiguous;
    args.qy = g.qy;
    args.insts = g.insts;
    args.stages = g.stages;
    args.ytile_bytes = g.ytile;
    // neighbouring tiles share X lines (segmented) or all of X (split b)
    args.xcd_remap = (g.contiguous && g.bsplit == 1) ? 0 : 1;
    args.vec_a = g.dt % 4 == 0 ? 1 : 0;
    args.bsplit = g.bsplit;
    args.b = f.s.b;
    args.xmap = g.xmap;
    args.yc = g.yc;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (f.xt == kF32 && f.wt == kF32) return launch_types<float, float>(f, g, args, grid);
    if (f.xt == kBF16 && f.wt == kBF16) return launch_types<bf16_t, bf16_t>(f, g, args, grid);
    if (f.xt == kF32 && f.wt == kBF16) return launch_types<float, bf16_t>(f, g, args, grid);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
