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
// weights (at most 64 KB a workgroup) are read once per workgroup, from the
// L2 cache after the first. fp32 accumulation; intermediates are fp32 (bf16 X
// and weights are widened exactly).
//
// Rows wider than the LDS allows are cut by the closure of the run. Factor
// (a, b, c, d) maps the slab alpha of a row (c*d inputs) to the slab alpha of
// the output (b*d values), and never changes an index modulo d. If P divides
// every a of the run and Q every d, the run therefore acts on each of P
// contiguous slabs of the row, and within a slab on each of Q classes of
// indices that are equal modulo Q, independently: on slab p, class q the
// factor is the KS factor (a/P, b, c, d/Q) with the blocks
// K[p*(a/P) + alpha'][delta'*Q + q]. A workgroup takes one slab and T
// consecutive classes (T divides Q) and keeps them with class fastest:
// tile element e*T + t is slab element e*Q + q0 + t, so on the tile each
// factor is again a KS factor, (a/P, b, c, (d/Q)*T), whose block
// (alpha', delta'') is K[p*(a/P) + alpha'][(delta''/T)*Q + q0 + delta''%T].
// X and Y move in runs of T elements. When a whole slab fits, a tile is
// instead consecutive slabs, as many as stay within a small width (P taken
// as a smaller divisor, Q = T = 1): one contiguous run, on which each factor
// is (a/P, b, c, d). The tile choice is run_tile below.
//
// Square factors run in place in one LDS buffer. Class tiles of short
// radix-2 runs take a persistent form that keeps each thread's blocks in
// registers across row blocks (tile_chain_persistent_kernel). Runs that are
// a whole radix-2/4 butterfly on every slab of 1024 or 4096 values, and
// whole-row butterflies, go to the register-resident kernel
// (ks_resident.hip), and other whole-row power-of-two runs to the
// digit-pass kernel (ks_digitchain.hip).

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;              // threads of a workgroup on whole rows
constexpr int kTiledThreads = 512;         // and on tiles of rows too wide for LDS
constexpr int kMaxFactors = 16;              // factors per launch
constexpr int kMaxWidth = 4096;              // widest row of the run (elements)
constexpr int kLdsTarget = 32 * 1024;        // LDS of the two row buffers (rows of 4096: 2 rows)
constexpr int kTiledLdsTarget = 48 * 1024;   // the same for tiles of rows too wide for LDS (three a CU)
constexpr int kMaxRows = 32;                 // rows per workgroup of a tiled run
constexpr int kMaxWholeRows = 256;           // and of a run on whole rows (narrow rows: many a workgroup)
constexpr int64_t kSlabTarget = 256;         // slabs merged into tiles of at most this many values
constexpr int64_t kClassWidth = 1024;        // widest tile made of index classes (12 rows in 48 KB)
constexpr int64_t kMaxWeightBytes = 64 * 1024;
constexpr int kMaxBlock = 16;                // b * c held in registers

constexpr int kMinRun = 32;                  // elements per run of X / Y when tiles are class groups

struct RowChainArgs {
    int nf;                  // factors in the run
    int pitch;               // LDS floats per row (widest tile row, multiple of 4)
    int rows;                // rows per workgroup
    int n_in, n_out;         // row widths of X and Y
    int64_t batch;
    int vec_x, vec_y;        // 1: tile rows of X / Y move as 4-element vectors
    int inplace;             // 1: every factor square on the register path, one LDS buffer
    int P, Q, T;             // slabs, classes per slab, classes per tile (T divides Q)
    int ntiles;              // P * (Q / T) tiles per row
    int tin, tout;           // tile widths of X and Y: (n_in / (P Q)) T, (n_out / (P Q)) T
    int pat[kMaxFactors][4]; // (a, b, c, d) of each factor
    int sub[kMaxFactors][2]; // (a / P, (d / Q) T): the factor on a tile
    const void* w[kMaxFactors];
};

// Where a tile's factor finds its blocks: tile group (alpha', delta'') is
// block (abase + alpha') * d + (delta'' / T) * Q + q0 + delta'' % T.
struct BlockMap {
    int abase, d, Q, T, q0;
    __device__ __forceinline__ int64_t block(int alpha, int dext) const {
        if (T == 1) return int64_t(abase + alpha) * d + dext * Q + q0;   // whole rows and slabs: no division
        const int dq = dext / T;
        return int64_t(abase + alpha) * d + dq * Q + q0 + (dext - dq * T);
    }
};

// Offset within a row of the tile element l (slab p, classes q0 ..): the
// slab's element (l / T) * Q + q0 + l % T; the slab itself when T = Q = 1.
__device__ __forceinline__ int tile_offset(int l, int slab0, int Q, int T, int q0) {
    if (T == Q) return slab0 + l;
    const int e = l / T;
    return slab0 + e * Q + q0 + (l - e * T);
}

// Threads of one factor (NT in the workgroup): with at least NT groups a
// thread takes groups t, t + NT, ... over all rows; with fewer, the rows of
// a group are dealt out to NT / groups threads.
struct ItemMap {
    int g0, gstep, r0, rstep;
};

template <int NT>
__device__ __forceinline__ bool item_map(int groups, ItemMap* m) {
    const int t = threadIdx.x;
    if (groups >= NT) {
        *m = ItemMap{t, NT, 0, 1};
        return true;
    }
    const int tpg = NT / groups;
    *m = ItemMap{t % groups, groups, t / groups, tpg};
    return t / groups < tpg;
}

// One factor from src to dst (rows [0, nr) of the workgroup) with B x C
// blocks: a thread holds the B * C weights of its (alpha, delta) group in
// registers and applies them to each of its rows (C inputs read from LDS
// once, B outputs written).
template <int NT, int B, int C, typename TW>
__device__ __forceinline__ void apply_block(const float* src, float* dst, int pitch, int nr, int a, int d,
                                            const TW* __restrict__ K, const BlockMap& bm) {
    // on tiles, the blocks of NB groups are loaded together (one wait on the
    // cache for NB groups, not one per group), at most 16 weights and 8
    // groups a thread; on whole rows one group at a time measured faster
    constexpr int NB = (NT != kTiledThreads || B * C >= 16) ? 1 : (16 / (B * C) > 8 ? 8 : 16 / (B * C));
    ItemMap m;
    if (!item_map<NT>(a * d, &m)) return;
    const int groups = a * d;
    for (int g0 = m.g0; g0 < groups; g0 += NB * m.gstep) {
        float w[NB][B][C];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int g = g0 + j * m.gstep;
            if (g < groups) {
                const int alpha = g / d;
                const TW* kp = K + bm.block(alpha, g - alpha * d) * (B * C);
#pragma unroll
                for (int be = 0; be < B; ++be)
#pragma unroll
                    for (int gm = 0; gm < C; ++gm) w[j][be][gm] = to_f32(kp[be * C + gm]);
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int g = g0 + j * m.gstep;
            if (g >= groups) break;
            const int alpha = g / d;
            const int delta = g - alpha * d;
            // with B == C the outputs land on the inputs' own places: each
            // thread reads all C inputs of a row before it writes, so src may
            // be dst
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
                    for (int gm = 0; gm < C; ++gm) acc = fmaf(w[j][be][gm], x[gm], acc);
                    o[r * pitch + be * d] = acc;
                }
            }
        }
    }
}

// Any b, c (up to 16): weights read from global memory (cached) per row.
template <int NT, typename TW>
__device__ __forceinline__ void apply_any(const float* src, float* dst, int pitch, int nr, int a, int b, int c,
                                          int d, const TW* __restrict__ K, const BlockMap& bm) {
    ItemMap m;
    if (!item_map<NT>(a * d, &m)) return;
    for (int g = m.g0; g < a * d; g += m.gstep) {
        const int alpha = g / d;
        const int delta = g - alpha * d;
        const TW* kp = K + bm.block(alpha, delta) * b * c;
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
template <int NT, int MAXBC, int B, int C, typename TW>
__device__ __forceinline__ bool try_block(const float* src, float* dst, int pitch, int nr, int a, int d,
                                          const TW* __restrict__ K, const BlockMap& bm) {
    if constexpr (B * C <= MAXBC) {
        apply_block<NT, B, C>(src, dst, pitch, nr, a, d, K, bm);
        return true;
    } else {
        return false;
    }
}

template <int NT, int MAXBC, int B, typename TW>
__device__ __forceinline__ void apply_b(const float* src, float* dst, int pitch, int nr, int a, int c, int d,
                                        const TW* __restrict__ K, const BlockMap& bm) {
    bool done = false;
    switch (c) {
        case 1: done = try_block<NT, MAXBC, B, 1>(src, dst, pitch, nr, a, d, K, bm); break;
        case 2: done = try_block<NT, MAXBC, B, 2>(src, dst, pitch, nr, a, d, K, bm); break;
        case 4: done = try_block<NT, MAXBC, B, 4>(src, dst, pitch, nr, a, d, K, bm); break;
        case 8: done = try_block<NT, MAXBC, B, 8>(src, dst, pitch, nr, a, d, K, bm); break;
        case 16: done = try_block<NT, MAXBC, B, 16>(src, dst, pitch, nr, a, d, K, bm); break;
    }
    if (!done) apply_any<NT>(src, dst, pitch, nr, a, B, c, d, K, bm);
}

// One factor on the tile: a and d are the tile's (a / P, (d / Q) T); bm
// finds the blocks.
template <int NT, int MAXBC, typename TW>
__device__ __forceinline__ void apply_factor(const float* src, float* dst, int pitch, int nr, int a, int b, int c,
                                             int d, const TW* __restrict__ K, const BlockMap& bm) {
    switch (b) {
        case 1: apply_b<NT, MAXBC, 1>(src, dst, pitch, nr, a, c, d, K, bm); return;
        case 2: apply_b<NT, MAXBC, 2>(src, dst, pitch, nr, a, c, d, K, bm); return;
        case 4: apply_b<NT, MAXBC, 4>(src, dst, pitch, nr, a, c, d, K, bm); return;
        case 8: apply_b<NT, MAXBC, 8>(src, dst, pitch, nr, a, c, d, K, bm); return;
        case 16: apply_b<NT, MAXBC, 16>(src, dst, pitch, nr, a, c, d, K, bm); return;
    }
    apply_any<NT>(src, dst, pitch, nr, a, b, c, d, K, bm);
}

// The X tile of rows [n0, n0 + nr) into LDS at z (bf16 widened exactly).
template <int NT, typename TX>
__device__ __forceinline__ void load_tile(const TX* __restrict__ X, float* z, const RowChainArgs& args, int64_t n0,
                                          int nr, int p, int q0) {
    const int t = threadIdx.x;
    const int pitch = args.pitch;
    const TX* xs = X + n0 * args.n_in;
    const int slab_in = p * (args.n_in / args.P);
    if (args.vec_x) {
        const int q = args.tin / 4;
        for (int i = t; i < nr * q; i += NT) {
            const int r = i / q, j = i - r * q;
            float v[4];
            load4_f32(xs + int64_t(r) * args.n_in + tile_offset(4 * j, slab_in, args.Q, args.T, q0), v);
            *reinterpret_cast<floatx4_t*>(z + r * pitch + 4 * j) = floatx4_t{v[0], v[1], v[2], v[3]};
        }
    } else {
        for (int i = t; i < nr * args.tin; i += NT) {
            const int r = i / args.tin, j = i - r * args.tin;
            z[r * pitch + j] = to_f32(xs[int64_t(r) * args.n_in + tile_offset(j, slab_in, args.Q, args.T, q0)]);
        }
    }
}

// The Y tile of rows [n0, n0 + nr) from LDS at z.
template <int NT>
__device__ __forceinline__ void store_tile(float* __restrict__ Y, const float* z, const RowChainArgs& args,
                                           int64_t n0, int nr, int p, int q0) {
    const int t = threadIdx.x;
    const int pitch = args.pitch;
    float* ys = Y + n0 * args.n_out;
    const int slab_out = p * (args.n_out / args.P);
    if (args.vec_y) {
        const int q = args.tout / 4;
        for (int i = t; i < nr * q; i += NT) {
            const int r = i / q, j = i - r * q;
            const floatx4_t v = *reinterpret_cast<const floatx4_t*>(z + r * pitch + 4 * j);
            __builtin_nontemporal_store(
                v, reinterpret_cast<floatx4_t*>(ys + int64_t(r) * args.n_out +
                                                tile_offset(4 * j, slab_out, args.Q, args.T, q0)));
        }
    } else {
        for (int i = t; i < nr * args.tout; i += NT) {
            const int r = i / args.tout, j = i - r * args.tout;
            ys[int64_t(r) * args.n_out + tile_offset(j, slab_out, args.Q, args.T, q0)] = z[r * pitch + j];
        }
    }
}

template <typename TX, typename TW, int MAXBC, int NT>
__global__ __launch_bounds__(NT) void row_chain_kernel(const TX* __restrict__ X, float* __restrict__ Y,
                                                             RowChainArgs args) {
    extern __shared__ __align__(16) float zbuf[];
    const int pitch = args.pitch;
    // buffers as offsets from the LDS array itself (a pointer picked from an
    // array of pointers would lose its address space: generic accesses)
    const int bufsz = args.inplace ? 0 : args.rows * pitch;
    const unsigned wg = blockIdx.x;
    // workgroup: row block, then tile (slab p, classes q0 .. q0 + T - 1)
    const int tile = static_cast<int>(wg % static_cast<unsigned>(args.ntiles));
    const int64_t n0 = int64_t(wg / static_cast<unsigned>(args.ntiles)) * args.rows;
    const int groups_per_slab = args.Q / args.T;
    const int p = tile / groups_per_slab;
    const int q0 = (tile - p * groups_per_slab) * args.T;
    const int nr = static_cast<int>(min(int64_t(args.rows), args.batch - n0));

    load_tile<NT>(X, zbuf, args, n0, nr, p, q0);
    __syncthreads();

    for (int f = 0; f < args.nf; ++f) {
        const int b = args.pat[f][1], c = args.pat[f][2];
        const int a = args.sub[f][0], d = args.sub[f][1];
        const BlockMap bm{p * a, args.pat[f][3], args.Q, args.T, q0};
        const TW* K = static_cast<const TW*>(args.w[f]);
        const float* src = zbuf + (f & 1) * bufsz;
        float* dst = zbuf + ((f + 1) & 1) * bufsz;
        apply_factor<NT, MAXBC>(src, dst, pitch, nr, a, b, c, d, K, bm);
        __syncthreads();
    }

    // the last buffer to Y
    store_tile<NT>(Y, zbuf + (args.nf & 1) * bufsz, args, n0, nr, p, q0);
}

// Tiles of index classes of a run of square radix-B factors (at most NF of
// them), when no factor has more (alpha, delta) groups on the
// tile than the workgroup has threads: a persistent workgroup keeps one
// tile and walks its row blocks (blockIdx / tiles, + gridDim / tiles, ...),
// holding the blocks of its group in every factor in registers for the
// whole launch instead of reading them again for every row block. Factors
// run in place.
template <typename TX, typename TW, int B, int NF>
__global__ __launch_bounds__(kTiledThreads) void tile_chain_persistent_kernel(const TX* __restrict__ X,
                                                                              float* __restrict__ Y,
                                                                              RowChainArgs args, int row_blocks) {
    constexpr int NT = kTiledThreads;
    extern __shared__ __align__(16) float zbuf[];
    const int pitch = args.pitch;
    const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(args.ntiles));
    const int first = static_cast<int>(blockIdx.x / static_cast<unsigned>(args.ntiles));
    const int step = static_cast<int>(gridDim.x / static_cast<unsigned>(args.ntiles));
    const int groups_per_slab = args.Q / args.T;
    const int p = tile / groups_per_slab;
    const int q0 = (tile - p * groups_per_slab) * args.T;

    // this thread's group in each factor (at most one: groups <= NT), its
    // rows (all, or every rstep-th when the groups are fewer than threads)
    // and the group's B x B block
    float w[NF][B][B];
    int off[NF], r0[NF], rstep[NF];
    bool has[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        has[f] = false;
        off[f] = 0;
        r0[f] = 0;
        rstep[f] = 1;
        if (f < args.nf) {
            const int a = args.sub[f][0], d = args.sub[f][1];
            ItemMap m;
            if (item_map<NT>(a * d, &m) && m.g0 < a * d) {
                const int alpha = m.g0 / d, delta = m.g0 - alpha * d;
                const BlockMap bm{p * a, args.pat[f][3], args.Q, args.T, q0};
                const TW* kp = static_cast<const TW*>(args.w[f]) + bm.block(alpha, delta) * (B * B);
#pragma unroll
                for (int be = 0; be < B; ++be)
#pragma unroll
                    for (int gm = 0; gm < B; ++gm) w[f][be][gm] = to_f32(kp[be * B + gm]);
                has[f] = true;
                off[f] = alpha * B * d + delta;
                r0[f] = m.r0;
                rstep[f] = m.rstep;
            }
        }
    }

    for (int rb = first; rb < row_blocks; rb += step) {
        const int64_t n0 = int64_t(rb) * args.rows;
        const int nr = static_cast<int>(min(int64_t(args.rows), args.batch - n0));
        __syncthreads();                          // the previous block's stores have read the tile
        load_tile<NT>(X, zbuf, args, n0, nr, p, q0);
        __syncthreads();
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f < args.nf) {
                if (has[f]) {
                    const int d = args.sub[f][1];
                    float* z = zbuf + off[f];
                    for (int r = r0[f]; r < nr; r += rstep[f]) {
                        float x[B];
#pragma unroll
                        for (int gm = 0; gm < B; ++gm) x[gm] = z[r * pitch + gm * d];
#pragma unroll
                        for (int be = 0; be < B; ++be) {
                            float acc = 0.0f;
#pragma unroll
                            for (int gm = 0; gm < B; ++gm) acc = fmaf(w[f][be][gm], x[gm], acc);
                            z[r * pitch + be * d] = acc;
                        }
                    }
                }
                __syncthreads();
            }
        }
        store_tile<NT>(Y, zbuf, args, n0, nr, p, q0);
    }
}

// Rows per workgroup: the row buffers (one when factors run in place, else
// two) in kLdsTarget bytes, kTiledLdsTarget for tiles of rows too wide for LDS (a
// tile's weights are read once per workgroup: more rows share them); at
// least two rows, so that each weight block loaded serves more than one row.
int chain_rows(int pitch, int nbuf, bool tiled) {
    const int target = tiled ? kTiledLdsTarget : kLdsTarget;
    return std::max(2, std::min(tiled ? kMaxRows : kMaxWholeRows, target / (nbuf * 4 * pitch)));
}

// Factors that can run in place: square blocks on the register path.
bool runs_in_place(const Shape* s, int n) {
    for (int k = 0; k < n; ++k)
        if (s[k].b != s[k].c || s[k].b * s[k].c > kMaxBlock || (s[k].b != 1 && s[k].b != 2 && s[k].b != 4))
            return false;
    return true;
}

int64_t gcd64(int64_t x, int64_t y) {
    while (y != 0) {
        const int64_t r = x % y;
        x = y;
        y = r;
    }
    return x;
}

// The tile a workgroup keeps in LDS: whole rows when the widest row of the
// run fits; else, with P = gcd of the a's, if one slab fits: consecutive
// slabs, as many as stay within kSlabTarget values (one when a slab is
// wider), a run of contiguous values; else one of the P slabs and T of its Q
// classes (Q = gcd of the d's), the most classes within kClassWidth values
// and at least kMinRun of them, so that fp32 X and Y move in runs of whole
// 128-byte lines (runs of 64 bytes read 1.5 times the bytes of X and Y by
// the HBM counters: each line fetched twice).
// Narrow tiles leave room for more rows, and every row a workgroup holds
// shares the weights it reads (measured on 65,536-, 16,384- and 8,192-point
// radix-2 and radix-4 butterflies: tiles of 256-value slabs and of 1024
// class values with up to 32 rows beat 4096-value tiles of 4 rows by up to
// 1.6 times; 512 threads and 48 KB of LDS a workgroup beat 256 threads and
// 64 KB by another 1.1 to 1.5 times, 1024 threads lost).
struct RunTile {
    int P, Q, T;
    int64_t width;           // floats of the widest tile row
};

bool run_tile(const Shape* s, int n, RunTile* rt) {
    int64_t w = s[0].n_in, P = 0, Q = 0;
    for (int k = 0; k < n; ++k) {
        w = std::max<int64_t>(w, s[k].n_out);
        P = gcd64(P, s[k].a);
        Q = gcd64(Q, s[k].d);
    }
    if (w <= kMaxWidth) {
        *rt = RunTile{1, 1, 1, w};
        return true;
    }
    if (w / P <= kMaxWidth) {
        int64_t slabs = P;
        for (int64_t f = 1; f <= P; ++f)
            if (P % f == 0 && w / f <= kSlabTarget) {
                slabs = f;
                break;
            }
        *rt = RunTile{static_cast<int>(slabs), 1, 1, w / slabs};
        return true;
    }
    const int64_t sub = w / (P * Q);
    int64_t T = 0;
    for (int64_t t = kClassWidth / sub; t >= kMinRun; --t)
        if (Q % t == 0) {
            T = t;
            break;
        }
    if (T == 0) return false;
    *rt = RunTile{static_cast<int>(P), static_cast<int>(Q), static_cast<int>(T), sub * T};
    return true;
}

int row_pitch(const RunTile& rt) { return static_cast<int>((rt.width + 3) / 4 * 4); }

}  // namespace

bool row_chain_supports(const Shape* s, int n, int xt, int wt) {
    (void)xt;
    if (n < 2 || n > kMaxFactors) return false;
    RunTile rt;
    if (!run_tile(s, n, &rt)) return false;
    for (int k = 0; k < n; ++k) {
        // small blocks only: with b * c = 64 the run measured no faster than one
        // launch per factor, with 128 2.4 times slower (VALU work and VGPRs)
        if (s[k].b * s[k].c > kMaxBlock) return false;
        // the blocks one workgroup reads for its tile
        if (s[k].nnz / (int64_t(rt.P) * rt.Q) * rt.T * elem_bytes(wt) > kMaxWeightBytes) return false;
    }
    return true;
}

// The persistent form takes class tiles of runs of at most 6 square radix-2
// factors with no more groups per factor on the tile than threads. Measured
// (4,096 rows of 65,536, 16,384 of 16,384): radix-2 class launches 0.53 ->
// 0.43 ms and 0.41 -> 0.37 ms; a radix-4 one (two factors) 0.45 -> 0.52 ms,
// so radix-4 keeps the per-block form.
constexpr int kPersistentFactors = 6;

bool persistent_tiles(const Shape* s, int n, const RunTile& rt) {
    if (rt.Q == 1) return false;          // whole rows and slabs
    if (n > kPersistentFactors) return false;
    for (int k = 0; k < n; ++k) {
        if (s[k].b != 2 || s[k].c != 2) return false;
        const int64_t groups = int64_t(s[k].a / rt.P) * (s[k].d / rt.Q * rt.T);
        if (groups > kTiledThreads) return false;
    }
    return true;
}

template <typename TX, typename TW>
ks_status_t launch_pt(dim3 grid, size_t lds, hipStream_t stream, const void* X, float* Y, const RowChainArgs& args,
                      int row_blocks) {
    const TX* x = static_cast<const TX*>(X);
    return launch_kernel(tile_chain_persistent_kernel<TX, TW, 2, kPersistentFactors>, grid, dim3(kTiledThreads), lds,
                         stream, x, Y, args, row_blocks);
}

template <typename TX, typename TW>
ks_status_t launch_rc(int maxbc, bool tiled, dim3 grid, size_t lds, hipStream_t stream, const void* X, float* Y,
                      const RowChainArgs& args) {
    const TX* x = static_cast<const TX*>(X);
    if (maxbc > kMaxBlock) return KS_ERR_UNSUPPORTED;
    if (tiled)
        return launch_kernel(row_chain_kernel<TX, TW, kMaxBlock, kTiledThreads>, grid, dim3(kTiledThreads), lds,
                             stream, x, Y, args);
    return launch_kernel(row_chain_kernel<TX, TW, kMaxBlock, kThreads>, grid, dim3(kThreads), lds, stream, x, Y,
                         args);
}

ks_status_t launch_row_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X, float* Y,
                             int64_t batch, hipStream_t stream, int num_cus) {
    if (!row_chain_supports(s, n, xt, wt)) return KS_ERR_UNSUPPORTED;
    RunTile rt;
    run_tile(s, n, &rt);
    const bool whole_rows = rt.P == 1 && rt.Q == 1;
    if (whole_rows && resident_chain_supports(s, n, xt, wt) && resident_chain_aligned(X, Y))
        return launch_resident_chain(s, n, xt, wt, W, X, Y, batch, stream, num_cus);
    // slabs that each carry a whole radix-2/4 butterfly of 1024 or 4096 values
    int rslabs = 0;
    if (!whole_rows && rt.Q == 1 && resident_slab_form(s, n, xt, wt, &rslabs) && resident_chain_aligned(X, Y))
        return launch_resident_slabs(s, n, rslabs, xt, wt, W, X, Y, batch, stream, num_cus);
    if (whole_rows && digit_chain_supports(s, n, xt, wt))
        return launch_digit_chain(s, n, xt, wt, W, X, Y, batch, stream);
    RowChainArgs args{};
    args.nf = n;
    args.pitch = row_pitch(rt);
    args.inplace = runs_in_place(s, n) ? 1 : 0;
    const int nbuf = args.inplace ? 1 : 2;
    args.rows = chain_rows(args.pitch, nbuf, !whole_rows);
    args.n_in = static_cast<int>(s[0].n_in);
    args.n_out = static_cast<int>(s[n - 1].n_out);
    args.batch = batch;
    args.P = rt.P;
    args.Q = rt.Q;
    args.T = rt.T;
    args.ntiles = rt.P * (rt.Q / rt.T);
    const int pq = rt.P * rt.Q;
    args.tin = args.n_in / pq * rt.T;
    args.tout = args.n_out / pq * rt.T;
    // 4-element vectors: every tile row starts on a multiple of 4 elements and
    // its runs are whole vectors (one run, the slab, when Q = 1; else runs of T)
    const uintptr_t xa = reinterpret_cast<uintptr_t>(X), ya = reinterpret_cast<uintptr_t>(Y);
    const int xvec_align = xt == kBF16 ? 8 : 16;
    const bool runs4 = rt.T == rt.Q || rt.T % 4 == 0;
    args.vec_x = (runs4 && args.n_in % 4 == 0 && (args.n_in / rt.P) % 4 == 0 && args.tin % 4 == 0 &&
                  xa % xvec_align == 0) ? 1 : 0;
    args.vec_y = (runs4 && args.n_out % 4 == 0 && (args.n_out / rt.P) % 4 == 0 && args.tout % 4 == 0 &&
                  ya % 16 == 0) ? 1 : 0;
    int maxbc = 1;
    for (int k = 0; k < n; ++k) {
        args.pat[k][0] = s[k].a;
        args.pat[k][1] = s[k].b;
        args.pat[k][2] = s[k].c;
        args.pat[k][3] = s[k].d;
        args.sub[k][0] = s[k].a / rt.P;
        args.sub[k][1] = s[k].d / rt.Q * rt.T;
        args.w[k] = W[k];
        maxbc = std::max(maxbc, s[k].b * s[k].c);
    }
    const int64_t blocks = (batch + args.rows - 1) / args.rows * args.ntiles;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const size_t lds = size_t(nbuf) * args.rows * args.pitch * 4;
    if (persistent_tiles(s, n, rt)) {
        // three workgroups a compute unit (48 KB of LDS each), the same number on every tile
        const int row_blocks = static_cast<int>((batch + args.rows - 1) / args.rows);
        const int64_t per_tile =
            std::max<int64_t>(1, std::min<int64_t>(row_blocks, int64_t(3) * std::max(1, num_cus) / args.ntiles));
        const dim3 pgrid(static_cast<unsigned>(per_tile * args.ntiles));
        if (xt == kF32 && wt == kF32) return launch_pt<float, float>(pgrid, lds, stream, X, Y, args, row_blocks);
        if (xt == kBF16 && wt == kBF16)
            return launch_pt<bf16_t, bf16_t>(pgrid, lds, stream, X, Y, args, row_blocks);
        if (xt == kF32 && wt == kBF16) return launch_pt<float, bf16_t>(pgrid, lds, stream, X, Y, args, row_blocks);
        return KS_ERR_UNSUPPORTED;
    }
    const dim3 grid(static_cast<unsigned>(blocks));
    if (xt == kF32 && wt == kF32) return launch_rc<float, float>(maxbc, !whole_rows, grid, lds, stream, X, Y, args);
    if (xt == kBF16 && wt == kBF16) return launch_rc<bf16_t, bf16_t>(maxbc, !whole_rows, grid, lds, stream, X, Y, args);
    if (xt == kF32 && wt == kBF16) return launch_rc<float, bf16_t>(maxbc, !whole_rows, grid, lds, stream, X, Y, args);
    return KS_ERR_UNSUPPORTED;
}

int row_chain_describe(const Shape* s, int n, char* buf, size_t len) {
    RunTile rt;
    if (!run_tile(s, n, &rt)) return std::snprintf(buf, len, "row-resident chain: unsupported");
    const bool whole_rows = rt.P == 1 && rt.Q == 1;
    if (whole_rows && resident_chain_supports(s, n, kF32, kF32)) return resident_chain_describe(s, n, 1, buf, len);
    int rslabs = 0;
    if (!whole_rows && rt.Q == 1 && resident_slab_form(s, n, kF32, kF32, &rslabs))
        return resident_chain_describe(s, n, rslabs, buf, len);
    if (whole_rows && digit_chain_supports(s, n, kF32, kF32)) return digit_chain_describe(s, n, buf, len);
    const int pitch = row_pitch(rt);
    const int nbuf = runs_in_place(s, n) ? 1 : 2;
    const int rows = chain_rows(pitch, nbuf, !whole_rows);
    if (whole_rows)
        return std::snprintf(buf, len, "row-resident chain: %d factors, rows/wg=%d, row pitch %d floats, %s, lds=%d",
                             n, rows, pitch, nbuf == 1 ? "in place" : "two buffers", nbuf * rows * pitch * 4);
    if (rt.Q == 1)
        return std::snprintf(buf, len,
                             "tile-resident chain: %d factors, %d slabs of %d values, rows/wg=%d, tile pitch %d "
                             "floats, %s, lds=%d",
                             n, rt.P, static_cast<int>(rt.width), rows, pitch, nbuf == 1 ? "in place" : "two buffers",
                             nbuf * rows * pitch * 4);
    return std::snprintf(buf, len,
                         "tile-resident chain: %d factors, %d slabs x %d classes, %d classes a tile, rows/wg=%d, "
                         "tile pitch %d floats, %s%s, lds=%d",
                         n, rt.P, rt.Q, rt.T, rows, pitch, nbuf == 1 ? "in place" : "two buffers",
                         persistent_tiles(s, n, rt) ? ", persistent (weights in registers)" : "",
                         nbuf * rows * pitch * 4);
}

}  // namespace ks
