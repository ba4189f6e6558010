// ks_valu.hip -- KS matmul for small blocks (b, c in {4, 8, 16}) on the
// vector ALUs.
//
// Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
//                                    * X[n][alpha][gamma][delta]
// (KS abstract page, taxoreview.com "dblp:303/4794", first paragraph). With
// b, c <= 16 the contraction is a few fp32 FMAs per output and the op is
// bound by HBM traffic, so the design goal is to move X and Y exactly once,
// in full cache lines, with no permutation pass (the same page, third
// sentence: a fused, output-stationary kernel).
//
// Workgroup tile: a set of (alpha, delta) pairs (all beta) and a range of
// rows. Every thread owns NB outputs of each row for a FIXED (alpha, delta)
// set, so its NB x c weights are loaded into registers once and reused for
// every row the workgroup streams (weight-stationary, output-stationary).
//
// X: the tile's part of each row is copied global -> LDS with 16-byte loads
// that cover whole segments, double-buffered across row steps (the global
// loads of step s+1 are in flight while step s computes). Threads then read
// X from LDS in whatever order the contraction wants.
//
// Two thread mappings:
//  * lane mode (d >= 8): lanes run over consecutive (alpha, delta) pairs,
//    delta fastest; a thread reads one X value per gamma and writes NB
//    outputs, each store coalesced across lanes along delta.
//  * slab mode (d in {1, 2, 4}): a thread owns an alpha' and all d deltas;
//    it reads the contiguous c*d slab of its alpha with 16-byte LDS reads and
//    writes NB*d contiguous outputs.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"

namespace ks {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 2;   // rows per double-buffered step

struct ValuArgs {
    int a, d;
    int64_t n_in, n_out;
    int64_t batch;
    int at;              // alphas per tile
    int dt;              // deltas per tile (lane mode), d in slab mode
    int tiles_delta;     // delta tiles per alpha tile
    int n_tiles;         // alpha tiles * delta tiles
    int steps_per_split; // row steps per workgroup
    int lds_row_bytes;   // LDS bytes per staged row
    int lds_alpha_bytes; // LDS bytes between alpha' slabs (contiguous chunks)
    int contiguous;      // 1: the tile's row chunk is one contiguous run
};

// Betas per thread. A thread holds NB*c*dv weights and prefetches kRows rows
// of its share of X (c*dv*G/... per row, see VPT), which together must stay
// near 176 registers so two waves fit per SIMD: the smallest power-of-two
// number of beta groups G with (b + kRows) * c * dv / G <= 176. The host
// planner uses the same rule.
__host__ __device__ constexpr int nb_rule(int b, int c, int dv) {
    int g = 1;
    while (g < b && (b + kRows) * c * dv > 176 * g) g *= 2;
    return b / g;
}

template <typename TX, typename TW, int B, int C, int DV, bool LANE>
__global__ __launch_bounds__(kThreads, 2) void valu_kernel(const TX* __restrict__ X,
                                                          const TW* __restrict__ K,
                                                          float* __restrict__ Y,
                                                          ValuArgs args) {
    constexpr int VW = 16 / int(sizeof(TX));                    // elements per 16-byte vector
    constexpr int NB = nb_rule(B, C, LANE ? 1 : DV);
    constexpr int G = B / NB;                                   // beta groups
    constexpr int P = kThreads / G;                             // pairs (lane) or alphas (slab)
    constexpr int R = kRows;                                    // rows per step
    constexpr int DVX = LANE ? 1 : DV;                          // deltas per thread
    // 16-byte vectors of X per row that each thread copies.
    constexpr int VPT = LANE ? (P * C / VW + kThreads - 1) / kThreads
                             : (P * C * DV / VW + kThreads - 1) / kThreads;
    static_assert(B % NB == 0, "beta groups must divide b");
    static_assert(VPT >= 1, "at least one vector per thread");

    extern __shared__ __align__(16) unsigned char lds[];

    const int t = threadIdx.x;
    const int tile = blockIdx.x % args.n_tiles;
    const int split = blockIdx.x / args.n_tiles;
    const int ta = tile / args.tiles_delta;
    const int td = tile - ta * args.tiles_delta;
    const int alpha0 = ta * args.at;
    const int delta0 = td * args.dt;
    const int d = args.d;

    // ---- thread -> (alpha', delta', beta group) -------------------------
    int g, al_l, de_l;
    if (LANE) {
        g = t / P;
        const int p = t - g * P;
        al_l = p / args.dt;
        de_l = p - al_l * args.dt;
        if (al_l >= args.at) al_l = args.at;  // marks the thread idle below
    } else {
        g = t % G;
        al_l = t / G;
        de_l = 0;
    }
    const int alpha = alpha0 + al_l;
    const int delta = delta0 + de_l;
    const bool active = (al_l < args.at) && alpha < args.a && (LANE ? (delta < d) : true);

    // ---- weights into registers: kr[j][dv][gamma] ------------------------
    float kr[NB][DVX][C];
    if (active) {
#pragma unroll
        for (int dv = 0; dv < DVX; ++dv) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const TW* kp = K + ((int64_t(alpha) * d + delta + dv) * B + g * NB + j) * C;
#pragma unroll
                for (int gm = 0; gm < C; ++gm) kr[j][dv][gm] = to_f32(kp[gm]);
            }
        }
    } else {
#pragma unroll
        for (int dv = 0; dv < DVX; ++dv)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int gm = 0; gm < C; ++gm) kr[j][dv][gm] = 0.0f;
    }

    // ---- the copy plan: which 16-byte vectors of each row this thread moves
    int64_t chunk_base;   // element offset of the tile's chunk within a row
    int at_eff = min(args.at, args.a - alpha0);
    int dt_eff = LANE ? min(args.dt, d - delta0) : DV;
    if (args.contiguous) chunk_base = int64_t(alpha0) * C * d;
    else chunk_base = int64_t(alpha0) * C * d + delta0;
    int gofs[VPT];
    int lofs[VPT];
    bool vok[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int q = t + i * kThreads;
        if (args.contiguous) {
            const int per_alpha = C * d / VW;       // vectors per alpha slab
            const int al = q / per_alpha;
            const int rem = q - al * per_alpha;
            gofs[i] = q * VW;
            lofs[i] = al * args.lds_alpha_bytes + rem * 16;
            vok[i] = al < at_eff && al < args.at;
        } else {
            const int per_seg = args.dt / VW;       // vectors per gamma segment
            const int gm = q / per_seg;
            const int e = q - gm * per_seg;
            gofs[i] = gm * d + e * VW;
            lofs[i] = (gm * args.dt + e * VW) * int(sizeof(TX));
            vok[i] = gm < C && e * VW < dt_eff;
        }
    }

    // ---- rows of this workgroup -------------------------------------------
    const int64_t row_begin = int64_t(split) * args.steps_per_split * R;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.steps_per_split) * R);
    const int nsteps = static_cast<int>((row_end - row_begin + R - 1) / R);

    const int buf_bytes = R * args.lds_row_bytes;
    u32x4 pre[R][VPT];

    auto load_step = [&](int s) {
        const int64_t n0 = row_begin + int64_t(s) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool row_ok = n0 + r < row_end;
            const TX* xrow = X + (n0 + r) * args.n_in + chunk_base;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                if (row_ok && vok[i]) pre[r][i] = *reinterpret_cast<const u32x4*>(xrow + gofs[i]);
            }
        }
    };
    auto store_lds = [&](int buf) {
        unsigned char* base = lds + buf * buf_bytes;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < VPT; ++i)
                if (vok[i]) *reinterpret_cast<u32x4*>(base + r * args.lds_row_bytes + lofs[i]) = pre[r][i];
    };

    load_step(0);
    store_lds(0);
    __syncthreads();

    // Output and LDS read offsets of this thread.
    const int64_t yoff = LANE ? (int64_t(alpha) * B + g * NB) * d + delta
                              : (int64_t(alpha) * B + g * NB) * DV;
    // Idle threads read a valid LDS address (their result is never stored).
    const int xl_off = !active ? 0
                     : LANE ? (args.contiguous ? al_l * args.lds_alpha_bytes + de_l * int(sizeof(TX))
                                               : de_l * int(sizeof(TX)))
                            : al_l * args.lds_alpha_bytes;
    const int gstride = LANE ? (args.contiguous ? d : args.dt) * int(sizeof(TX)) : 0;

    for (int s = 0; s < nsteps; ++s) {
        if (s + 1 < nsteps) load_step(s + 1);
        const unsigned char* base = lds + (s & 1) * buf_bytes;
        const int64_t n0 = row_begin + int64_t(s) * R;
#pragma unroll 1
        for (int r = 0; r < R; ++r) {
            const unsigned char* xr = base + r * args.lds_row_bytes + xl_off;
            float acc[NB][DVX];
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int dv = 0; dv < DVX; ++dv) acc[j][dv] = 0.0f;
            if (LANE) {
#pragma unroll
                for (int gm = 0; gm < C; ++gm) {
                    const float x = to_f32(*reinterpret_cast<const TX*>(xr + gm * gstride));
#pragma unroll
                    for (int j = 0; j < NB; ++j) acc[j][0] = fmaf(kr[j][0][gm], x, acc[j][0]);
                }
            } else {
                // The slab holds c*DV elements, element e = gamma*DV + delta.
#pragma unroll
                for (int v = 0; v < C * DV / VW; ++v) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(xr + v * 16);
                    float xv[VW];
                    if (sizeof(TX) == 4) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) xv[e] = __uint_as_float(w[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            xv[2 * e] = bf16_lo(w[e]);
                            xv[2 * e + 1] = bf16_hi(w[e]);
                        }
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
            const int64_t n = n0 + r;
            if (active && n < row_end) {
                float* yrow = Y + n * args.n_out + yoff;
                if (LANE) {
#pragma unroll
                    for (int j = 0; j < NB; ++j) yrow[int64_t(j) * d] = acc[j][0];
                } else {
                    constexpr int NOUT = NB * DVX;
                    if (NOUT % 4 == 0) {
#pragma unroll
                        for (int v = 0; v < NOUT / 4; ++v) {
                            float4 o;
                            o.x = acc[(4 * v + 0) / DVX][(4 * v + 0) % DVX];
                            o.y = acc[(4 * v + 1) / DVX][(4 * v + 1) % DVX];
                            o.z = acc[(4 * v + 2) / DVX][(4 * v + 2) % DVX];
                            o.w = acc[(4 * v + 3) / DVX][(4 * v + 3) % DVX];
                            reinterpret_cast<float4*>(yrow)[v] = o;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < NOUT; ++e) yrow[e] = acc[e / DVX][e % DVX];
                    }
                }
            }
        }
        if (s + 1 < nsteps) store_lds((s + 1) & 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Host side: tile geometry and dispatch.

struct ValuGeom {
    bool lane;
    int nb, g, p, at, dt, tiles_delta, n_tiles, contiguous;
    int lds_row_bytes, lds_alpha_bytes, vw, r;
};

int nb_for(int b, int c, int dv) { return nb_rule(b, c, dv); }

bool geom_for(const Shape& s, int xt, ValuGeom* gm) {
    const int eb = elem_bytes(xt);
    const int vw = 16 / eb;
    const int b = s.b, c = s.c, d = s.d;
    if (!((b == 4 || b == 8 || b == 16) && (c == 4 || c == 8 || c == 16))) return false;
    gm->vw = vw;
    gm->r = kRows;
    if (d >= 8) {
        if (d % vw != 0) return false;
        gm->lane = true;
        gm->nb = nb_for(b, c, 1);
        gm->g = b / gm->nb;
        gm->p = kThreads / gm->g;
        if (d >= gm->p) {
            gm->dt = gm->p;
            gm->at = 1;
            gm->contiguous = 0;
            gm->lds_row_bytes = c * gm->dt * eb;
            gm->lds_alpha_bytes = gm->lds_row_bytes;
        } else {
            gm->dt = d;
            gm->at = gm->p / d;
            gm->contiguous = 1;
            // alpha' stride congruent to d words mod 64 banks (lanes reading
            // consecutive (alpha', delta) then hit distinct banks), rounded to
            // keep 16-byte alignment.
            const int slab = c * d * eb;
            int stride = slab;
            const int want = (d * eb) % 256;
            while ((stride % 256) != want || stride % 16 != 0) stride += 16;
            gm->lds_alpha_bytes = stride;
            gm->lds_row_bytes = gm->at * stride;
        }
    } else {
        if (d != 1 && d != 2 && d != 4) return false;
        if ((c * d) % vw != 0) return false;
        gm->lane = false;
        gm->nb = nb_for(b, c, d);
        gm->g = b / gm->nb;
        gm->p = kThreads / gm->g;
        gm->at = gm->p;
        gm->dt = d;
        gm->contiguous = 1;
        const int slab = c * d * eb;
        // odd multiple of 16 bytes: 16 consecutive alpha' slabs start in
        // distinct 16-byte bank groups.
        gm->lds_alpha_bytes = (slab % 32 == 0) ? slab + 16 : slab;
        gm->lds_row_bytes = gm->at * gm->lds_alpha_bytes;
    }
    const int tiles_alpha = (s.a + gm->at - 1) / gm->at;
    gm->tiles_delta = gm->lane ? (d + gm->dt - 1) / gm->dt : 1;
    if (gm->contiguous) gm->tiles_delta = 1;
    const int64_t nt = int64_t(tiles_alpha) * gm->tiles_delta;
    if (nt > (int64_t(1) << 30)) return false;
    gm->n_tiles = static_cast<int>(nt);
    return true;
}

template <typename TX, typename TW, int B, int C>
ks_status_t launch_bc(const FactorCall& f, const ValuGeom& gm, const ValuArgs& args, dim3 grid) {
    const size_t lds = size_t(2) * gm.r * gm.lds_row_bytes;
    const TX* X = static_cast<const TX*>(f.X);
    const TW* K = static_cast<const TW*>(f.W);
    if (gm.lane) {
        hipLaunchKernelGGL((valu_kernel<TX, TW, B, C, 1, true>), grid, dim3(kThreads), lds, f.stream, X, K, f.Y, args);
    } else if (f.s.d == 1) {
        hipLaunchKernelGGL((valu_kernel<TX, TW, B, C, 1, false>), grid, dim3(kThreads), lds, f.stream, X, K, f.Y, args);
    } else if (f.s.d == 2) {
        hipLaunchKernelGGL((valu_kernel<TX, TW, B, C, 2, false>), grid, dim3(kThreads), lds, f.stream, X, K, f.Y, args);
    } else {
        hipLaunchKernelGGL((valu_kernel<TX, TW, B, C, 4, false>), grid, dim3(kThreads), lds, f.stream, X, K, f.Y, args);
    }
    return hipGetLastError() == hipSuccess ? KS_OK : KS_ERR_HIP;
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

void split_rows(const ValuGeom& gm, int64_t batch, int num_cus, int rows_per_block,
                int* row_splits, int* steps_per_split) {
    const int64_t steps_total = (batch + gm.r - 1) / gm.r;
    int64_t splits;
    if (rows_per_block > 0) {
        const int64_t spb = std::max<int64_t>(1, (rows_per_block + gm.r - 1) / gm.r);
        splits = (steps_total + spb - 1) / spb;
    } else {
        // About eight workgroups per compute unit in total, but at least
        // 32 row steps (128 rows) per workgroup so the weight load amortises.
        const int64_t want = int64_t(std::max(num_cus, 1)) * 8;
        splits = std::max<int64_t>(1, want / std::max(gm.n_tiles, 1));
        splits = std::min(splits, std::max<int64_t>(1, steps_total / 32));
    }
    splits = std::max<int64_t>(1, std::min(splits, steps_total));
    const int64_t spp = (steps_total + splits - 1) / splits;
    splits = (steps_total + spp - 1) / spp;
    *row_splits = static_cast<int>(splits);
    *steps_per_split = static_cast<int>(spp);
}

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
    int splits = 0, spp = 0;
    split_rows(gm, batch, num_cus, 0, &splits, &spp);
    return std::snprintf(buf, len,
                         "valu %s: nb=%d groups=%d alphas/tile=%d deltas/tile=%d tiles=%d "
                         "row_splits=%d rows/wg=%d lds=%d",
                         gm.lane ? "lane" : "slab", gm.nb, gm.g, gm.at, gm.dt, gm.n_tiles, splits,
                         spp * gm.r, 2 * gm.r * gm.lds_row_bytes);
}

ks_status_t launch_valu(const FactorCall& f) {
    ValuGeom gm;
    if (!geom_for(f.s, f.xt, &gm)) return KS_ERR_UNSUPPORTED;
    if (!aligned16(f.X) || !aligned16(f.W) || !aligned16(f.Y)) return KS_ERR_UNSUPPORTED;
    if ((f.s.n_in * elem_bytes(f.xt)) % 16 != 0 || (f.s.n_out * 4) % 16 != 0) return KS_ERR_UNSUPPORTED;
    int splits = 0, spp = 0;
    split_rows(gm, f.batch, f.num_cus, f.rows_per_block, &splits, &spp);
    const int64_t blocks = int64_t(gm.n_tiles) * splits;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
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
    args.steps_per_split = spp;
    args.lds_row_bytes = gm.lds_row_bytes;
    args.lds_alpha_bytes = gm.lds_alpha_bytes;
    args.contiguous = gm.contiguous;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (f.xt == kF32 && f.wt == kF32) return launch_types<float, float>(f, gm, args, grid);
    if (f.xt == kBF16 && f.wt == kBF16) return launch_types<bf16_t, bf16_t>(f, gm, args, grid);
    if (f.xt == kF32 && f.wt == kBF16) return launch_types<float, bf16_t>(f, gm, args, grid);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace ks
