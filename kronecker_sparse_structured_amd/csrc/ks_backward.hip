// ks_backward.hip -- gradients of one KS factor, for a layer's backward pass.
//
// For Y = X * W^T with W's support I_a (x) 1_{b x c} (x) I_d (KS abstract
// page, taxoreview.com "dblp:303/4794", first paragraph) and dY = dL/dY:
//   dX = dY * W. W^T is again a KS matrix, of pattern (a, c, b, d) with every
//        b x c block transposed, so dX is the forward product of that
//        pattern; this file only transposes the blocks (nnz elements, into
//        the caller's workspace) and the forward kernels do the rest.
//   dK[alpha][delta][beta][gamma] = sum_n dY[n][alpha][beta][delta]
//                                         * X[n][alpha][gamma][delta]
//        (each K entry sits in W once). Blocks with b and c multiples of 16
//        run on the matrix cores (below); any other pattern on a generic
//        kernel that gives every thread one K entry. Both write partial sums
//        per range of rows to the workspace, which a second kernel adds in
//        range order, so the result does not depend on scheduling.

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <vector>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

constexpr int kThreads = 256;

// Wt[blk][gamma][beta] = W[blk][beta][gamma] for blk < a*d.
template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_blocks_kernel(const T* __restrict__ W, T* __restrict__ Wt, int b,
                                                                    int c, int64_t nnz) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;   // index into Wt
    if (e >= nnz) return;
    const int64_t bc = int64_t(b) * c;
    const int64_t blk = e / bc;
    const int r = static_cast<int>(e - blk * bc);
    const int gamma = r / b, beta = r - gamma * b;
    Wt[e] = W[blk * bc + int64_t(beta) * c + gamma];
}

// One K entry per thread (gamma fastest, as K is stored), rows
// [split * rows_per_split, ...) of the batch; writes its partial sum to
// out[split * nnz + entry] (out is dK itself when there is one split).
template <typename TX>
__global__ __launch_bounds__(kThreads) void dw_generic_kernel(const float* __restrict__ dY, const TX* __restrict__ X,
                                                              float* __restrict__ out, int a, int b, int c, int d,
                                                              int64_t batch, int64_t rows_per_split, int64_t nnz) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (e >= nnz) return;
    const int gamma = static_cast<int>(e % c);
    int64_t q = e / c;
    const int beta = static_cast<int>(q % b);
    q /= b;
    const int delta = static_cast<int>(q % d);
    const int alpha = static_cast<int>(q / d);
    const int64_t n_in = int64_t(a) * c * d, n_out = int64_t(a) * b * d;
    const int64_t n0 = int64_t(blockIdx.y) * rows_per_split;
    const int64_t n1 = min(batch, n0 + rows_per_split);
    const float* gy = dY + (int64_t(alpha) * b + beta) * d + delta;
    const TX* gx = X + (int64_t(alpha) * c + gamma) * d + delta;
    float acc = 0.0f;
    for (int64_t n = n0; n < n1; ++n) acc = fmaf(gy[n * n_out], to_f32(gx[n * n_in]), acc);
    out[int64_t(blockIdx.y) * nnz + e] = acc;
}

// Small blocks (b, c in {2, 4, 8, 16}, not both 16): one (alpha, delta)
// block per thread with its b x c sums in registers, rows
// [split * rows_per_split, ...). Per row a thread loads the block's b
// values of dY and c values of X once (lanes run over delta, then alpha, so
// the loads of a wave are runs of consecutive elements), so the kernel
// reads each element of dY and X once per row range.
template <typename TX, int B, int C>
__global__ __launch_bounds__(kThreads) void dw_small_kernel(const float* __restrict__ dY, const TX* __restrict__ X,
                                                            float* __restrict__ out, int a, int d, int64_t batch,
                                                            int64_t rows_per_split, int64_t nnz) {
    const int64_t blk = int64_t(blockIdx.x) * kThreads + threadIdx.x;   // alpha * d + delta
    if (blk >= int64_t(a) * d) return;
    const int alpha = static_cast<int>(blk / d);
    const int delta = static_cast<int>(blk - int64_t(alpha) * d);
    const int64_t n_in = int64_t(a) * C * d, n_out = int64_t(a) * B * d;
    const int64_t n0 = int64_t(blockIdx.y) * rows_per_split;
    const int64_t n1 = min(batch, n0 + rows_per_split);
    const float* gy = dY + int64_t(alpha) * B * d + delta;      // + beta * d
    const TX* gx = X + int64_t(alpha) * C * d + delta;          // + gamma * d
    float acc[B][C];
#pragma unroll
    for (int i = 0; i < B; ++i)
#pragma unroll
        for (int j = 0; j < C; ++j) acc[i][j] = 0.0f;
    for (int64_t n = n0; n < n1; ++n) {
        float yv[B], xv[C];
#pragma unroll
        for (int i = 0; i < B; ++i) yv[i] = gy[n * n_out + i * d];
#pragma unroll
        for (int j = 0; j < C; ++j) xv[j] = to_f32(gx[n * n_in + j * d]);
#pragma unroll
        for (int i = 0; i < B; ++i)
#pragma unroll
            for (int j = 0; j < C; ++j) acc[i][j] = fmaf(yv[i], xv[j], acc[i][j]);
    }
    float* o = out + int64_t(blockIdx.y) * nnz + blk * (B * C);   // dK[alpha][delta][beta][gamma]
#pragma unroll
    for (int i = 0; i < B; ++i)
#pragma unroll
        for (int j = 0; j < C; ++j) o[i * C + j] = acc[i][j];
}

// dK[e] = sum of part[s * nnz + e] over the splits s: a workgroup takes 64
// entries, each with four threads that add a quarter of the splits in
// ascending order; the quarters are then added in order (0 + 1) + (2 + 3),
// so the result does not depend on scheduling.
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(const float* __restrict__ part, float* __restrict__ dK,
                                                             int nsplit, int64_t nnz) {
    __shared__ float q[4][64];
    const int lane = threadIdx.x & 63, qi = threadIdx.x >> 6;
    const int64_t e = int64_t(blockIdx.x) * 64 + lane;
    const int per = (nsplit + 3) / 4;
    const int s0 = qi * per, s1 = min(nsplit, s0 + per);
    float acc = 0.0f;
    if (e < nnz)
        for (int s = s0; s < s1; ++s) acc += part[int64_t(s) * nnz + e];
    q[qi][lane] = acc;
    __syncthreads();
    if (qi == 0 && e < nnz) dK[e] = (q[0][lane] + q[1][lane]) + (q[2][lane] + q[3][lane]);
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (e < n) p[e] = 0.0f;
}

unsigned grid_for(int64_t n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }


// ---------------------------------------------------------------------------
// dK on the matrix cores, for blocks with b and c multiples of 16.
//
// For a fixed (alpha, delta), dK[alpha][delta] (b x c) = dY_blk^T X_blk summed
// over rows: M = beta, N = gamma, K = rows, four rows per
// v_mfma_f32_16x16x4_f32. A workgroup owns a tile -- one alpha, dt deltas
// (all d, or segments of dt), bt of the b outputs -- and a range of rows; one
// loader wave streams both the tile's part of X and of dY, 16 rows a stage,
// into an LDS ring (ks_stream.h); four compute waves keep the tile's
// dt * (bt / 16) * (c / 16) accumulator tiles (at most 64) in registers over
// all the rows, then write them as the range's partial sums. Rows past the
// batch in the last stage contribute zero (both operands are masked).

typedef float floatx4_dw __attribute__((ext_vector_type(4)));

constexpr int kDwRows = 16;          // rows per stage
constexpr int kDwMaxInsts = 40;      // loader instructions per stage, each of X and dY
constexpr int kDwTilesPerWave = 16;  // accumulator tiles per compute wave (64 VGPRs)

struct DwArgs {
    int a, b, c, d;
    int64_t n_in, n_out, batch;
    int bt, dt;                  // outputs and deltas per tile
    int tiles_beta, tiles_delta, n_tiles;
    int ntiles_acc;              // dt * (bt / 16) * (c / 16)
    int rows_per_split;          // multiple of kDwRows
    int contiguous;              // 1: dt == d (whole alpha slabs of X and of dY's beta range)
    int insts_x, insts_y, stages;
    StageMap xmap, ymap;
    int64_t out_stride;          // elements between the partial sums of consecutive splits (0: one split)
};

// NL loader waves: with two, each issues every other instruction of X's and
// of dY's part of a stage and waits on its own vector-memory counter, which
// doubles the loads a workgroup keeps in flight (a wave's counter allows 63).
template <typename TX, int NL>
__global__ __launch_bounds__(kConsumerThreads + 64 * NL) void dw_mfma_kernel(const float* __restrict__ dY,
                                                                              const TX* __restrict__ X,
                                                                              float* __restrict__ out, DwArgs args) {
    constexpr int EB = int(sizeof(TX));
    constexpr int VWX = 16 / EB;
    extern __shared__ __align__(16) unsigned char lds[];
    const int stage_bytes = (args.insts_x + args.insts_y) * 1024;
    const int t = threadIdx.x;
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int tile = blk % args.n_tiles;
    const int split = blk / args.n_tiles;
    const int tb = tile % args.tiles_beta;          // beta splits of one (alpha, delta range) are neighbours
    const int rest = tile / args.tiles_beta;
    const int td = rest % args.tiles_delta;
    const int alpha = rest / args.tiles_delta;
    const int beta0 = tb * args.bt;
    const int delta0 = td * args.dt;
    const int d = args.d;
    const bool contig = args.contiguous != 0;
    // the tile's part of a row: X[alpha][gamma][delta0 ..], dY[alpha][beta0 ..][delta0 ..]
    const int64_t xg0 = int64_t(alpha) * args.c * d + (contig ? 0 : delta0);
    const int64_t yg0 = (int64_t(alpha) * args.b + beta0) * d + (contig ? 0 : delta0);

    const int64_t row_begin = int64_t(split) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kDwRows - 1) / kDwRows);
    const int S = args.stages;

    if (t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        LoaderPlan<kDwMaxInsts> lx, ly;
        const int lane = t & 63;
        const int L = (t - kConsumerThreads) >> 6;             // loader wave
        make_loader_plan<kDwMaxInsts>(args.xmap, args.insts_x, VWX, EB, args.n_in, args.xmap.blocks,
                                      args.xmap.blk_vec, lane, &lx);
        make_loader_plan<kDwMaxInsts>(args.ymap, args.insts_y, 4, 4, args.n_out, args.ymap.blocks,
                                      args.ymap.blk_vec, lane, &ly);
        // this wave's instructions per stage
        const int own = (args.insts_x - L + NL - 1) / NL + (args.insts_y - L + NL - 1) / NL;
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kDwRows;
            unsigned char* st = lds + (s % S) * stage_bytes;
            if constexpr (NL == 1) {
                issue_stage<kDwMaxInsts>(lx, args.insts_x, X + n0 * args.n_in + xg0,
                                         stage_limit(n0, row_end, args.n_in, EB), st);
                issue_stage<kDwMaxInsts>(ly, args.insts_y, dY + n0 * args.n_out + yg0,
                                         stage_limit(n0, row_end, args.n_out, 4), st + args.insts_x * 1024);
            } else {
                issue_stage_part<kDwMaxInsts>(lx, args.insts_x, X + n0 * args.n_in + xg0,
                                              stage_limit(n0, row_end, args.n_in, EB), st, L, NL);
                issue_stage_part<kDwMaxInsts>(ly, args.insts_y, dY + n0 * args.n_out + yg0,
                                              stage_limit(n0, row_end, args.n_out, 4), st + args.insts_x * 1024, L,
                                              NL);
            }
        };
        for (int s = 0; s < S - 1 && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            wait_vmcnt_upto(min(63, min(S - 2, nsteps - 1 - s) * own));
            lds_barrier();                                   // stage s ready
            if (s + S - 1 < nsteps) issue(s + S - 1);
            lds_barrier();                                   // stage s consumed
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + i][l % 16] in register i.
    // A = dY^T (M = beta, K = row), B = X (K = row, N = gamma).
    const int w = t >> 6;
    const int lane = t & 63;
    const int mn = lane & 15;
    const int kk = lane >> 4;
    const int MT = args.bt / 16, NT = args.c / 16;
    const int xs = contig ? d : args.dt;                     // element stride of gamma in an X stage row
    const int ys = contig ? d : args.dt;                     // element stride of beta in a dY stage row
    const int xrow = args.xmap.row_vec * 16, yrow = args.ymap.row_vec * 16;
    int aoff[kDwTilesPerWave], boff[kDwTilesPerWave];       // byte offsets within a stage row
    // this wave's tiles w, w + 4, ..: the first `ntv` of its slots
    const int ntv = __builtin_amdgcn_readfirstlane((args.ntiles_acc - w + 3) / 4);
#pragma unroll
    for (int j = 0; j < kDwTilesPerWave; ++j) {
        const int ti = w + 4 * j;
        const int dl = ti / (MT * NT);
        const int mt = (ti / NT) % MT;
        const int nt = ti % NT;
        aoff[j] = ((16 * mt + mn) * ys + dl) * 4;
        boff[j] = ((16 * nt + mn) * xs + dl) * EB;
    }
    floatx4_dw acc[kDwTilesPerWave];
#pragma unroll
    for (int j = 0; j < kDwTilesPerWave; ++j) acc[j] = floatx4_dw{0.0f, 0.0f, 0.0f, 0.0f};

    for (int s = 0; s < nsteps; ++s) {
        lds_barrier();                                                   // stage s ready
        const unsigned char* xst = lds + (s % S) * stage_bytes;
        const unsigned char* yst = xst + args.insts_x * 1024;
        const int rows = static_cast<int>(min(int64_t(kDwRows), row_end - row_begin - int64_t(s) * kDwRows));
#pragma unroll
        for (int ks = 0; ks < kDwRows / 4; ++ks) {
            const int r = 4 * ks + kk;
            const bool rv = r < rows;
            const unsigned char* yr = yst + r * yrow;
            const unsigned char* xr = xst + r * xrow;
#pragma unroll
            for (int j = 0; j < kDwTilesPerWave; ++j) {
                if (j >= ntv) continue;
                const float av = rv ? *reinterpret_cast<const float*>(yr + aoff[j]) : 0.0f;
                const float bv = rv ? to_f32(*reinterpret_cast<const TX*>(xr + boff[j])) : 0.0f;
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
            }
        }
        lds_barrier();                                                   // stage s consumed
    }
    // partial sums of this row range: dK[alpha][delta][beta][gamma]
    float* o = out + int64_t(split) * args.out_stride;
#pragma unroll
    for (int j = 0; j < kDwTilesPerWave; ++j) {
        if (j >= ntv) continue;
        const int ti = w + 4 * j;
        const int dl = ti / (MT * NT);
        const int mt = (ti / NT) % MT;
        const int nt = ti % NT;
        const int gamma = 16 * nt + mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int beta = beta0 + 16 * mt + 4 * kk + i;
            o[((int64_t(alpha) * d + delta0 + dl) * args.b + beta) * args.c + gamma] = acc[j][i];
        }
    }
}


// Tile of the matrix-core dK kernel for pattern s and X element size eb.
struct DwGeom {
    int bt, dt, contiguous, tiles_beta, tiles_delta, n_tiles, ntiles_acc, insts_x, insts_y, stages, loaders;
    StageMap xmap, ymap;
    size_t lds;
};

// Odd number of 16-byte vectors per row: 16 rows start in distinct bank groups.
int odd_pitch(int vec) { return vec % 2 ? vec : vec + 1; }

bool dw_geom(const Shape& s, int xt, DwGeom* g) {
    const int b = s.b, c = s.c, d = s.d;
    if (b % 16 != 0 || c % 16 != 0) return false;
    const int eb = elem_bytes(xt), vwx = 16 / eb;
    const int nt = c / 16;
    auto finish = [&](int bt, int dt, bool contig) {
        g->bt = bt;
        g->dt = dt;
        g->contiguous = contig ? 1 : 0;
        g->tiles_beta = b / bt;
        g->tiles_delta = contig ? 1 : d / dt;
        const int64_t ntl = int64_t(s.a) * g->tiles_delta * g->tiles_beta;
        if (ntl > (int64_t(1) << 30)) return false;
        g->n_tiles = static_cast<int>(ntl);
        g->ntiles_acc = dt * (bt / 16) * nt;
        StageMap& xm = g->xmap;
        StageMap& ym = g->ymap;
        xm.rows = ym.rows = kDwRows;
        xm.pad_vec = ym.pad_vec = 0;
        if (contig) {
            xm.blocks = 1; xm.blk_vec = c * d / vwx; xm.gstride = 0;
            ym.blocks = 1; ym.blk_vec = bt * d / 4; ym.gstride = 0;
        } else {
            xm.blocks = c; xm.blk_vec = dt / vwx; xm.gstride = d;
            ym.blocks = bt; ym.blk_vec = dt / 4; ym.gstride = d;
        }
        xm.row_vec = odd_pitch(xm.blocks * xm.blk_vec);
        ym.row_vec = odd_pitch(ym.blocks * ym.blk_vec);
        g->insts_x = (kDwRows * xm.row_vec + 63) / 64;
        g->insts_y = (kDwRows * ym.row_vec + 63) / 64;
        const int insts = g->insts_x + g->insts_y;
        if (g->insts_x > kDwMaxInsts || g->insts_y > kDwMaxInsts || insts > 63) return false;
        // the loader addresses a stage with 32-bit byte offsets
        if (int64_t(kDwRows) * std::max(s.n_in * eb, s.n_out * 4) >= (int64_t(1) << 31)) return false;
        // A wave keeps at most 63 loads in flight. Where X arrives in short
        // runs (segments of under 64 bytes: many pieces a stage), a second
        // loader wave takes every other instruction and the ring deepens
        // (measured: (1,128,128,32) 711 -> 559 us on 16,384 rows); with
        // longer runs a second loader measured slower (ViT factor 83 -> 99 us).
        g->loaders = (!contig && dt * eb < 64 && insts > 21) ? 2 : 1;
        const int own = (g->insts_x + g->loaders - 1) / g->loaders + (g->insts_y + g->loaders - 1) / g->loaders;
        int st = std::max(3, std::min(8, (g->loaders == 2 ? 160 : 150) * 1024 / (insts * 1024)));
        while (st > 3 && (st - 2) * own > 63) --st;
        g->stages = st;
        g->lds = size_t(st) * insts * 1024;
        return g->lds <= 160 * 1024;
    };
    // whole alpha slabs when the accumulators of every delta fit
    for (int bt = b; bt >= 16; bt /= 2) {
        if (b % bt != 0 || bt % 16 != 0) continue;
        if (d * (bt / 16) * nt <= 4 * kDwTilesPerWave && (c * d * eb) % 16 == 0 && (bt * d * 4) % 16 == 0 &&
            finish(bt, d, true))
            return true;
    }
    // else segments of dt deltas (16-byte runs at least), longest first
    const int dtmin = std::max(4, vwx);
    for (int dt = 64; dt >= dtmin; dt /= 2) {
        if (d % dt != 0) continue;
        for (int bt = b; bt >= 16; bt /= 2) {
            if (b % bt != 0 || bt % 16 != 0) continue;
            if (dt * (bt / 16) * nt <= 4 * kDwTilesPerWave && finish(bt, dt, false)) return true;
        }
    }
    return false;
}

// The partial sums of every row range stay within this many bytes, so one
// array of this size serves any call as its workspace.
constexpr int64_t kDwPartialBytes = int64_t(64) << 20;
static_assert(kDwPartialBytes == KS_DW_SCRATCH_BYTES, "the documented scratch size");

// Row ranges: about 512 workgroups (a fixed target, so that the workspace
// size is known without asking the device), at most 256 ranges, partial
// sums within kDwPartialBytes.
int dw_ranges(const Shape& s, int64_t batch, int64_t tiles, int rows_step, int64_t target = 512) {
    const int64_t steps = (batch + rows_step - 1) / rows_step;
    int64_t r = std::max<int64_t>(1, target / std::max<int64_t>(tiles, 1));
    r = std::min<int64_t>(r, std::min<int64_t>(steps, 256));
    r = std::min<int64_t>(r, std::max<int64_t>(1, kDwPartialBytes / (s.nnz * 4)));
    return static_cast<int>(std::max<int64_t>(1, r));
}

// Scratch of ks_matmul_dw_noalloc: the dK partial sums of one call, for
// callers that cannot allocate. One copy per GPU, held until the process
// ends; calls on one GPU share it (each call writes every partial sum it
// reads, so nothing needs clearing between calls; calls that overlap in time
// on one GPU race).
static __device__ __align__(256) unsigned char scratch[kDwPartialBytes];

}  // namespace

size_t dw_scratch_bytes() { return static_cast<size_t>(kDwPartialBytes); }

// The device address of `scratch` on the current device. In host code the
// array's name is only a stand-in for the symbol, so kernels get this
// address instead; it is looked up once per device, with that device
// current.
ks_status_t dw_scratch(void** ptr) {
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KS_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= static_cast<int>(addr.size())) addr.resize(dev + 1, nullptr);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KS_ERR_HIP;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return KS_OK;
}

ks_status_t launch_transpose_blocks(const Shape& s, int wt, const void* W, void* Wt, hipStream_t stream) {
    if (grid_for(s.nnz) == 0) return KS_OK;
    if (wt == kF32)
        return launch_kernel(transpose_blocks_kernel<float>, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream,
                             static_cast<const float*>(W), static_cast<float*>(Wt), s.b, s.c, s.nnz);
    return launch_kernel(transpose_blocks_kernel<bf16_t>, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream,
                         static_cast<const bf16_t*>(W), static_cast<bf16_t*>(Wt), s.b, s.c, s.nnz);
}

// Plan of one dK call: the kernel family and its ranges of rows.
bool small_size(int v) { return v == 2 || v == 4 || v == 8 || v == 16; }

template <typename TX, int B, int C>
ks_status_t launch_small_bc(const Shape& s, const float* dY, const void* X, float* out, int64_t batch, int64_t rps,
                            int ranges, hipStream_t stream) {
    const dim3 grid(grid_for(int64_t(s.a) * s.d), static_cast<unsigned>(ranges));
    return launch_kernel(dw_small_kernel<TX, B, C>, grid, dim3(kThreads), 0, stream, dY, static_cast<const TX*>(X), out,
                         s.a, s.d, batch, rps, s.nnz);
}

template <typename TX, int B>
ks_status_t launch_small_b(const Shape& s, const float* dY, const void* X, float* out, int64_t batch, int64_t rps,
                           int ranges, hipStream_t stream) {
    switch (s.c) {
        case 2: return launch_small_bc<TX, B, 2>(s, dY, X, out, batch, rps, ranges, stream);
        case 4: return launch_small_bc<TX, B, 4>(s, dY, X, out, batch, rps, ranges, stream);
        case 8: return launch_small_bc<TX, B, 8>(s, dY, X, out, batch, rps, ranges, stream);
        case 16:
            if constexpr (B <= 8) return launch_small_bc<TX, B, 16>(s, dY, X, out, batch, rps, ranges, stream);
            break;
    }
    return KS_ERR_UNSUPPORTED;
}

template <typename TX>
ks_status_t launch_small_t(const Shape& s, const float* dY, const void* X, float* out, int64_t batch, int64_t rps,
                           int ranges, hipStream_t stream) {
    switch (s.b) {
        case 2: return launch_small_b<TX, 2>(s, dY, X, out, batch, rps, ranges, stream);
        case 4: return launch_small_b<TX, 4>(s, dY, X, out, batch, rps, ranges, stream);
        case 8: return launch_small_b<TX, 8>(s, dY, X, out, batch, rps, ranges, stream);
        case 16: return launch_small_b<TX, 16>(s, dY, X, out, batch, rps, ranges, stream);
    }
    return KS_ERR_UNSUPPORTED;
}

ks_status_t launch_small(const Shape& s, int xt, const float* dY, const void* X, float* out, int64_t batch,
                         int64_t rps, int ranges, hipStream_t stream) {
    if (xt == kF32) return launch_small_t<float>(s, dY, X, out, batch, rps, ranges, stream);
    return launch_small_t<bf16_t>(s, dY, X, out, batch, rps, ranges, stream);
}

struct DwPlan {
    bool mfma;
    bool small;      // dw_small_kernel
    DwGeom g;
    int ranges;
    int64_t rows_per_range;
};

DwPlan dw_plan(const Shape& s, int xt, int64_t batch) {
    DwPlan pl;
    pl.mfma = dw_geom(s, xt, &pl.g);
    pl.small = !pl.mfma && small_size(s.b) && small_size(s.c) && s.b * s.c <= 128;
    if (batch <= 1) {
        pl.ranges = 1;
    } else if (pl.mfma) {
        // one resident round of workgroups on a 256-unit device (a fixed
        // count keeps the workspace size device-independent)
        const int64_t per_cu = std::max<size_t>(1, std::min<size_t>(2, (160 * 1024) / pl.g.lds));
        pl.ranges = dw_ranges(s, batch, pl.g.n_tiles, kDwRows, 256 * per_cu);
    } else if (pl.small) {
        // about 64 K threads (one per block and row range)
        const int64_t blocks = int64_t(s.a) * s.d;
        pl.ranges = dw_ranges(s, batch, std::max<int64_t>(1, blocks * 512 / 65536), 1);
    } else {
        // generic: about 2048 workgroups of one K entry per thread
        const int64_t groups = (s.nnz + kThreads - 1) / kThreads;
        pl.ranges = dw_ranges(s, batch, std::max<int64_t>(1, groups / 4), 1);
    }
    const int step = pl.mfma ? kDwRows : 1;
    const int64_t steps = (batch + step - 1) / step;
    pl.rows_per_range = std::max<int64_t>(1, (steps + pl.ranges - 1) / pl.ranges) * step;
    if (batch > 0) pl.ranges = static_cast<int>((batch + pl.rows_per_range - 1) / pl.rows_per_range);
    return pl;
}

size_t dw_workspace_bytes(const Shape& s, int xt, int64_t batch) {
    const DwPlan pl = dw_plan(s, xt, batch);
    return pl.ranges <= 1 ? 0 : (static_cast<size_t>(pl.ranges) * s.nnz * 4 + 255) / 256 * 256;
}

ks_status_t launch_dw(const Shape& s, int xt, const float* dY, const void* X, float* dK, int64_t batch, void* ws,
                      hipStream_t stream) {
    if (batch == 0)
        return launch_kernel(fill_zero_kernel, dim3(grid_for(s.nnz)), dim3(kThreads), 0, stream, dK, s.nnz);
    const DwPlan pl = dw_plan(s, xt, batch);
    float* out = pl.ranges > 1 ? static_cast<float*>(ws) : dK;
    // The matrix-core kernel streams X and dY in 16-byte vectors; for
    // pointers aligned only to their element size the generic kernel runs
    // over the same row ranges, so the partial sums fit the same workspace.
    const bool vec_ok = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && (reinterpret_cast<uintptr_t>(dY) & 15u) == 0;
    ks_status_t st;
    if (pl.mfma && vec_ok) {
        DwArgs args;
        args.a = s.a; args.b = s.b; args.c = s.c; args.d = s.d;
        args.n_in = s.n_in; args.n_out = s.n_out; args.batch = batch;
        args.bt = pl.g.bt; args.dt = pl.g.dt;
        args.tiles_beta = pl.g.tiles_beta; args.tiles_delta = pl.g.tiles_delta; args.n_tiles = pl.g.n_tiles;
        args.ntiles_acc = pl.g.ntiles_acc;
        args.rows_per_split = static_cast<int>(pl.rows_per_range);
        args.contiguous = pl.g.contiguous;
        args.insts_x = pl.g.insts_x; args.insts_y = pl.g.insts_y; args.stages = pl.g.stages;
        args.xmap = pl.g.xmap; args.ymap = pl.g.ymap;
        args.out_stride = pl.ranges > 1 ? s.nnz : 0;
        const int64_t blocks = int64_t(pl.g.n_tiles) * pl.ranges;
        if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
        const dim3 grid(static_cast<unsigned>(blocks));
        const dim3 blk1(kConsumerThreads + 64), blk2(kConsumerThreads + 128);
        const float* xf = static_cast<const float*>(X);
        const bf16_t* xb = static_cast<const bf16_t*>(X);
        if (xt == kF32 && pl.g.loaders == 2)
            st = launch_kernel(dw_mfma_kernel<float, 2>, grid, blk2, pl.g.lds, stream, dY, xf, out, args);
        else if (xt == kF32)
            st = launch_kernel(dw_mfma_kernel<float, 1>, grid, blk1, pl.g.lds, stream, dY, xf, out, args);
        else if (pl.g.loaders == 2)
            st = launch_kernel(dw_mfma_kernel<bf16_t, 2>, grid, blk2, pl.g.lds, stream, dY, xb, out, args);
        else
            st = launch_kernel(dw_mfma_kernel<bf16_t, 1>, grid, blk1, pl.g.lds, stream, dY, xb, out, args);
    } else if (pl.small) {
        st = launch_small(s, xt, dY, X, out, batch, pl.rows_per_range, pl.ranges, stream);
    } else {
        const dim3 grid(grid_for(s.nnz), static_cast<unsigned>(pl.ranges));
        if (xt == kF32)
            st = launch_kernel(dw_generic_kernel<float>, grid, dim3(kThreads), 0, stream, dY,
                               static_cast<const float*>(X), out, s.a, s.b, s.c, s.d, batch, pl.rows_per_range, s.nnz);
        else
            st = launch_kernel(dw_generic_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, dY,
                               static_cast<const bf16_t*>(X), out, s.a, s.b, s.c, s.d, batch, pl.rows_per_range,
                               s.nnz);
    }
    if (st != KS_OK || pl.ranges == 1) return st;
    return launch_kernel(dw_reduce_kernel, dim3(static_cast<unsigned>((s.nnz + 63) / 64)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(ws), dK, pl.ranges, s.nnz);
}

int dw_describe(const Shape& s, int xt, int64_t batch, char* buf, size_t len) {
    const DwPlan pl = dw_plan(s, xt, batch);
    if (pl.small)
        return std::snprintf(buf, len, "dw small: one block per thread, ranges=%d", pl.ranges);
    if (!pl.mfma)
        return std::snprintf(buf, len, "dw generic: one K entry per thread, ranges=%d", pl.ranges);
    return std::snprintf(buf, len,
                         "dw mfma 16x16x4f32: deltas/tile=%d (%s) outputs/tile=%d of %d acc tiles=%d ranges=%d "
                         "rows/range=%lld wgs=%lld stages=%d x %d KB loaders=%d",
                         pl.g.dt, pl.g.contiguous ? "contiguous" : "segmented", pl.g.bt, s.b, pl.g.ntiles_acc,
                         pl.ranges, static_cast<long long>(pl.rows_per_range),
                         static_cast<long long>(int64_t(pl.g.n_tiles) * pl.ranges), pl.g.stages,
                         pl.g.insts_x + pl.g.insts_y, pl.g.loaders);
}

}  // namespace ks
