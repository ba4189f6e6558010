// ks_slab.hip -- two KS factors in one launch when the second one works
// inside the first one's output slabs.
//
// Butterfly-type layers are chains of KS factors (KS abstract page,
// taxoreview.com "dblp:303/4794", first paragraph). In a chain
// F = (a, 16, 16, 16) followed by G = (16a, 16, 16, 1) -- the last two
// factors of the 65,536-point butterfly -- F maps each alpha slab of a row
// of X (X[alpha][gamma][delta], 256 values) to an alpha slab of the
// intermediate Z[alpha][beta][delta], and G's input group alpha' =
// 16 alpha + beta is Z[alpha][beta][0..15]: it lies inside that slab. A
// workgroup that owns one alpha for a range of rows therefore reads only
// X's alpha slab (1 KB of fp32 per row), writes only Y's slab
// Y[16 alpha .. 16 alpha + 15][beta'] (another contiguous 1 KB per row),
// and needs 16 blocks of each factor's weights (32 KB of fp32). Z stays in
// LDS: the pair moves |X| + |Y| through HBM instead of |X| + 2|Z| + |Y|.
//
// Workgroup: one loader wave streams the rows' X slabs into an LDS ring
// (ks_stream.h), 16 rows a stage; four compute waves, per stage,
//  (A) compute Z for the stage's rows on the matrix cores: for a fixed
//      delta, Z[rows][beta][delta] = X[rows][.][delta] (16 x 16) times
//      K_F[alpha][delta] (16 x 16); wave w takes deltas 4w .. 4w + 3, whose
//      A operands one 16-byte LDS read supplies together;
//  (B) after an LDS barrier, compute Y from Z the same way: for a fixed
//      beta, Y[rows][16 alpha + beta][.] = Z[rows][beta][.] (16 x 16) times
//      K_G[16 alpha + beta][0]^T; wave w takes betas 4w .. 4w + 3;
// and a storer wave writes the previous stage's Y tile from the other of
// two LDS buffers as 16-byte vectors covering whole 1 KB row slabs.
//
// Alignment. X and Y need only be aligned to their element size. When X
// starts xshift elements past a 16-byte boundary, the loader streams the
// 16-byte granules that cover each slab from the boundary below it (a
// granule never crosses a page, so the extra bytes are always readable), one
// granule more per row (it takes the row's pad vector), and phase A reads
// single elements xshift places further on; when Y is not 16-byte aligned
// the storer writes single elements.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kN = 16;                 // b = c = d of F; b' = c' of G
constexpr int kSlab = kN * kN;         // elements of one alpha slab of X, Z and Y
constexpr int kR = 16;                 // rows per stage: one MFMA M tile
constexpr int kTileRow = kSlab + 4;    // LDS pitch (floats) of a row of the Z and Y tiles
constexpr int kTileFloats = kR * kTileRow;

// Loader instructions (1 KB each) per stage: 16 rows of one slab plus one
// pad vector per row (rows start in different banks).
__host__ __device__ constexpr int slab_stage_insts(int eb) { return (kR * (kSlab * eb / 16 + 1) + 63) / 64; }

struct SlabArgs {
    int a;                   // alphas of F
    int64_t n_in, n_out;     // a * 256 each
    int64_t batch;
    int rows_per_split;      // a multiple of kR
    int insts, stages;       // loader instructions per stage, ring depth
    StageMap xmap;           // LDS layout of an X stage
    int xshift;              // elements from the 16-byte boundary below X to X (the same in every row)
};

// kVec: X and Y are 16-byte aligned (xshift == 0): 16-byte LDS reads of X
// and 16-byte stores of Y.
template <typename TX, typename TW, bool kVec>
__global__ __launch_bounds__(kStreamThreads + 64) void slab_pair_kernel(const TX* __restrict__ X,
                                                                        const TW* __restrict__ KF,
                                                                        const TW* __restrict__ KG,
                                                                        float* __restrict__ Y, SlabArgs args) {
    constexpr int EB = int(sizeof(TX));
    constexpr int VW = 16 / EB;
    constexpr int kMaxInsts = slab_stage_insts(EB);
    static_assert(kMaxInsts <= 63, "vmcnt is six bits");
    extern __shared__ __align__(16) unsigned char lds[];
    const int kStageBytes = args.insts * 1024;
    const int kStages = args.stages;
    float* const zt = reinterpret_cast<float*>(lds + kStages * kStageBytes);   // Z tile [kR][kTileRow]
    float* const yt0 = zt + kTileFloats;                                         // 2 Y tiles [kR][kTileRow]
    const int xrow_bytes = args.xmap.row_vec * 16;

    const int t = threadIdx.x;
    const int alpha = static_cast<int>(blockIdx.x % static_cast<unsigned>(args.a));
    const int split = static_cast<int>(blockIdx.x / static_cast<unsigned>(args.a));
    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kR - 1) / kR);

    if (t >= kStreamThreads) {
        // ------------------------------------------------------ storer wave
        // issue priority over the compute waves sharing its SIMD, so the
        // stores drain while they run the MFMAs
        __builtin_amdgcn_s_setprio(3);
        const int lane = t & 63;
        auto store_tile = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const int rows = static_cast<int>(min(int64_t(kR), row_end - n0));
            const float* yt = yt0 + (s & 1) * kTileFloats + 4 * lane;
            float* yg = Y + n0 * args.n_out + int64_t(alpha) * kSlab + 4 * lane;
            floatx4 v[kR];
#pragma unroll
            for (int r = 0; r < kR; ++r) v[r] = *reinterpret_cast<const floatx4*>(yt + r * kTileRow);
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                if (r < rows) {
                    if constexpr (kVec) {
                        __builtin_nontemporal_store(v[r], reinterpret_cast<floatx4*>(yg + r * args.n_out));
                    } else {
#pragma unroll
                        for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[r][k], yg + r * args.n_out + k);
                    }
                }
            }
        };
        for (int s = 0; s < nsteps; ++s) {
            lds_barrier();                                   // stage s ready
            if (s > 0) store_tile(s - 1);
            lds_barrier();                                   // Z of stage s written
            lds_barrier();                                   // Y tile s written
        }
        store_tile(nsteps - 1);
        return;
    }

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        LoaderPlan<kMaxInsts> lp;
        make_loader_plan<kMaxInsts>(args.xmap, args.insts, VW, EB, args.n_in, 1, args.xmap.blk_vec,
                                    t - kConsumerThreads, &lp);
        const TX* xbase = X - args.xshift + int64_t(alpha) * kSlab;   // 16-byte aligned
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            // vectors at or past the end of the last row's slab (and the
            // granule holding its last elements, when shifted) load a dummy
            const int64_t end = ((row_end - n0 - 1) * args.n_in + kSlab) * EB + (args.xshift != 0 ? 16 : 0);
            const uint32_t limit = end >= int64_t(kNoVector) ? kNoVector : static_cast<uint32_t>(end);
            issue_stage<kMaxInsts>(lp, args.insts, xbase + n0 * args.n_in, limit, lds + (s % kStages) * kStageBytes);
        };
        for (int s = 0; s < kStages - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            wait_vmcnt_upto(min(kStages - 2, nsteps - 1 - s) * args.insts);
            lds_barrier();                                   // stage s ready
            if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
            lds_barrier();                                   // Z of stage s written
            lds_barrier();                                   // Y tile s written
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + i][l % 16] in register i.
    const int w = t >> 6;
    const int lane = t & 63;
    const int col = lane & 15;      // A: row; B, D: output column
    const int grp = lane >> 4;      // A, B: k within the step; D: group of 4 rows
    // (A) pairs delta = 4w + u; B = K_F[alpha][delta][beta = col][gamma = 4 ks + grp]
    float kf[4][4];
    // (B) pairs beta = 4w + u; B = K_G[16 alpha + beta][0][beta' = col][gamma' = 4 grp + ks]:
    // each lane's k group takes 4 consecutive gamma' so that one 16-byte
    // read of Z gives its A operands for all four steps
    float kg[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const TW* fp = KF + ((int64_t(alpha) * kN + 4 * w + u) * kN + col) * kN;
        const TW* gp = KG + ((int64_t(alpha) * kN + 4 * w + u) * kN + col) * kN;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kf[u][ks] = to_f32(fp[4 * ks + grp]);
            kg[u][ks] = to_f32(gp[4 * grp + ks]);
        }
    }

    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();                                                   // stage s ready
        const unsigned char* xs = lds + (s % kStages) * kStageBytes;
        // (A) Z[row][beta][delta] = sum_gamma K_F[alpha][delta][beta][gamma] X[row][alpha][gamma][delta]
        {
            const TX* xa = reinterpret_cast<const TX*>(xs + col * xrow_bytes) + args.xshift + grp * kN + 4 * w;
            floatx4 z[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) z[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float av[4];
                if constexpr (kVec) {
                    load4_f32(xa + ks * 4 * kN, av);                     // deltas 4w .. 4w + 3 of one gamma
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) av[u] = to_f32(xa[ks * 4 * kN + u]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) z[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], kf[u][ks], z[u], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<floatx4*>(zt + (4 * grp + i) * kTileRow + col * kN + 4 * w) =
                    floatx4{z[0][i], z[1][i], z[2][i], z[3][i]};
        }
        lds_barrier();                                                   // Z written
        // (B) Y[row][16 alpha + beta][beta'] = sum_gamma' K_G[16 alpha + beta][0][beta'][gamma'] Z[row][beta][gamma']
        {
            float* yt = yt0 + (s & 1) * kTileFloats;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const floatx4 zv = *reinterpret_cast<const floatx4*>(zt + col * kTileRow + (4 * w + u) * kN + 4 * grp);
                floatx4 y = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) y = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[ks], kg[u][ks], y, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) yt[(4 * grp + i) * kTileRow + (4 * w + u) * kN + col] = y[i];
            }
        }
        lds_barrier();                                                   // Y tile s written
    }
}

bool shape_ok(const Shape& s0, const Shape& s1) {
    return s0.b == kN && s0.c == kN && s0.d == kN && s1.a == int64_t(s0.a) * kN && s1.b == kN && s1.c == kN &&
           s1.d == 1;
}

template <typename TX, typename TW>
ks_status_t launch_typed(const Shape& s0, const void* W0, const void* W1, const void* X, float* Y, int64_t batch,
                         hipStream_t stream, int num_cus) {
    constexpr int EB = int(sizeof(TX));
    SlabArgs args;
    args.xshift = static_cast<int>((reinterpret_cast<uintptr_t>(X) & 15u) / EB);
    const bool vec = args.xshift == 0 && (reinterpret_cast<uintptr_t>(Y) & 15u) == 0;
    args.a = s0.a;
    args.n_in = s0.n_in;
    args.n_out = s0.n_out;
    args.batch = batch;
    args.xmap.rows = kR;
    args.xmap.blocks = 1;
    // one slab per row and one pad vector (rows start in different banks);
    // a shifted slab spans one granule more, which takes the pad vector
    args.xmap.blk_vec = kSlab * EB / 16 + (args.xshift != 0 ? 1 : 0);
    args.xmap.pad_vec = 0;
    args.xmap.row_vec = kSlab * EB / 16 + 1;
    args.xmap.gstride = 0;
    args.insts = slab_stage_insts(EB);
    // one workgroup per compute unit: the ring takes what the Z and Y tiles leave of ~150 KB
    const size_t tiles = size_t(3) * kTileFloats * sizeof(float);
    args.stages = static_cast<int>(std::max<size_t>(3, std::min<size_t>(6, (150 * 1024 - tiles) / (args.insts * 1024))));
    while (args.stages > 3 && (args.stages - 2) * args.insts > 63) --args.stages;   // the loader's vmcnt wait
    const size_t lds = size_t(args.stages) * args.insts * 1024 + tiles;
    // about one resident wave of workgroups, equal row shares
    const int64_t steps_total = (batch + kR - 1) / kR;
    const int64_t splits = std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) / args.a);
    const int64_t steps = std::max<int64_t>(1, (steps_total + splits - 1) / splits);
    args.rows_per_split = static_cast<int>(steps * kR);
    const int64_t nsplit = (batch + args.rows_per_split - 1) / args.rows_per_split;
    const int64_t blocks = nsplit * args.a;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    auto kernel = vec ? slab_pair_kernel<TX, TW, true> : slab_pair_kernel<TX, TW, false>;
    return launch_kernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads + 64), lds, stream,
                         static_cast<const TX*>(X), static_cast<const TW*>(W0), static_cast<const TW*>(W1), Y, args);
}

}  // namespace

bool slab_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1) {
    if (wt0 != wt1) return false;
    if (!((xt == kF32 && (wt0 == kF32 || wt0 == kBF16)) || (xt == kBF16 && wt0 == kBF16))) return false;
    if (!shape_ok(s0, s1)) return false;
    // the loader addresses a stage with 32-bit byte offsets
    return int64_t(kR) * s0.n_in * elem_bytes(xt) < (int64_t(1) << 31);
}

ks_status_t launch_slab_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                             const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                             int num_cus) {
    if (!slab_pair_supports(s0, s1, xt, wt0, wt1)) return KS_ERR_UNSUPPORTED;
    // X and Y aligned to their element size (checked by the caller); rows
    // are whole 16-byte granules apart, so every row has X's misalignment
    if ((reinterpret_cast<uintptr_t>(X) % elem_bytes(xt)) != 0 || (reinterpret_cast<uintptr_t>(Y) & 3u) != 0)
        return KS_ERR_UNSUPPORTED;
    if (xt == kF32 && wt0 == kF32) return launch_typed<float, float>(s0, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kBF16 && wt0 == kBF16) return launch_typed<bf16_t, bf16_t>(s0, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kF32 && wt0 == kBF16) return launch_typed<float, bf16_t>(s0, W0, W1, X, Y, batch, stream, num_cus);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
