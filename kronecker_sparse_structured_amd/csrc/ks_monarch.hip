// ks_monarch.hip -- a Monarch-shaped pair of KS factors in one launch:
// F = (M, N, N, 1), a block-diagonal factor of M blocks of N x N, then
// G = (1, M, M, N), which mixes the M blocks for each of the N positions.
//
// KS matrices underpin Butterfly and Monarch matrices (KS abstract page,
// taxoreview.com "dblp:303/4794", first paragraph, first sentence). A row of
// X is X[alpha][gamma] (M x N), F gives Z[alpha][beta] = sum_gamma
// K_F[alpha][0][beta][gamma] X[alpha][gamma], and G reads Z as
// Z[gamma' = alpha][delta' = beta] and gives Y[beta'][beta] = sum_alpha
// K_G[0][beta][beta'][alpha] Z[alpha][beta]. The pair mixes every value of a
// row, so a workgroup holds 16 whole rows (at most 4 KB each) in an LDS
// stage; the intermediate never leaves the chip and the pair moves
// |X| + |Y| + weights through HBM instead of |X| + 2 |Z| + |Y|.
//
// Every row needs all of the two factors' weights (M N N + N M M values),
// and each compute wave needs those of its own groups at every stage; they
// stay in registers for the whole launch: up to 96 a lane with four compute
// waves, and for M = N = 32 (256 KB of fp32, half a compute unit's register
// file) 64 a lane spread over sixteen waves. In both products
// the k index is assigned so that a lane's k values are consecutive (lane
// group g takes k = (K / 4) g + ks in step ks; any order of the k sum is the
// same sum up to rounding), which makes a lane's B operands of one group
// consecutive weights (16-byte loads) and its A operands consecutive values
// of the row.
//
// Per 16-row stage, in place in LDS (NW compute waves: four, or sixteen for
// 32 x 32 blocks):
//  (A) wave w takes the blocks alpha = w M / NW ..: Z[rows][alpha][beta] =
//      X[rows][alpha][.] (16 x N) times the block's transpose, written over
//      X[rows][alpha][.] (a wave reads and writes only its own blocks);
//  (B) after an LDS barrier, wave w takes positions beta = w N / NW .., four
//      (two with sixteen waves) at a time (one LDS read gives the A operands
//      of those positions): Y[rows][beta'][beta] = Z[rows][.][beta] (16 x M)
//      times K_G[beta]'s transpose, written over Z[rows][.][beta];
//  (C) after another barrier the compute waves store the rows.
// A loader wave streams the next stages from HBM meanwhile; sixteen compute
// waves fill a workgroup's 1024 threads, so there each copies its own share
// of the next stage.
//
// LDS row layout (floats): value (x, y) at x * (N + 4) + y, rows
// M (N + 4) + 4 apart: the 16 rows, the 16 consecutive y or the 16
// consecutive x that one instruction spreads its lanes over fall in
// different 16-byte bank groups. bf16 X lands in the first half of each
// index's slot (value (x, y) at byte 4 x (N + 4) + 2 y); phase A reads a
// block's inputs before it writes that block's fp32 results over the same
// slot. X and Y 16-byte aligned. The weights need only their element
// alignment: their 16-byte loads are valid at any such alignment in the
// unaligned-access mode that ROCm sets for this GPU family (the compiler
// merges element loads into the same instructions by itself).

#include <algorithm>
#include <type_traits>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kR = 16;                               // rows per stage: one MFMA M tile

// NW compute waves plus one loader wave (NW = 4), or sixteen compute waves
// that copy their own shares of the next stage (SELF: 32 x 32 blocks, whose
// weights the sixteen waves keep in registers between them).
template <int M, int N, int NW>
struct MonShape {
    static constexpr bool SELF = NW == 16;
    static constexpr int THREADS = NW * 64 + (SELF ? 0 : 64);
    static constexpr int CONSUMERS = NW * 64;
    static constexpr int XP = N + 4;                 // floats per index x in LDS
    static constexpr int RP = M * XP + 4;            // floats per row in LDS
    static constexpr int XVEC = N / 4;               // 16-byte vectors per x in a row of Y (fp32)
    static constexpr int STAGE_VEC = kR * RP / 4;    // 16-byte LDS vectors per stage
    static constexpr int INSTS = (STAGE_VEC + 63) / 64;
    static constexpr int STAGE_BYTES = INSTS * 1024;
    static constexpr int STAGES = std::min(4, (150 * 1024) / STAGE_BYTES);
    static constexpr int KSF = N / 4, NTF = N / 16;  // F: k steps (gamma), N tiles (beta)
    static constexpr int KSG = M / 4, NTG = M / 16;  // G: k steps (alpha), N tiles (beta')
    static constexpr int GA = M / NW;                // F blocks per wave
    static constexpr int GB = N / NW;                // G positions per wave
    static constexpr int BB = GB < 4 ? GB : 4;       // G positions a batch (one LDS read of Z)
    static_assert(GA >= 1 && GB % BB == 0 && (BB == 2 || BB == 4), "a wave takes whole batches of G positions");
    static_assert(STAGES >= 2 && (N == 16 || N == 32) && (M == 16 || M == 32), "shapes");
    static_assert(!SELF || STAGES == 2, "the self-copy waits assume two stages");
    static_assert(RP % 4 == 0 && (RP / 4) % 2 == 1 && XP % 4 == 0, "16-byte rows; odd row pitch in vectors");
};

struct MonArgs {
    int64_t n;               // row width M * N
    int64_t batch;
    int rows_per_split;      // a multiple of kR
};

// Four consecutive weights in registers: fp32 as loaded (16 bytes), bf16
// packed (8 bytes) and widened when used.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename TW> struct WReg { typedef floatx4 type; };
template <> struct WReg<bf16_t> { typedef u32x2 type; };

// count consecutive 4-value registers of weights from p (16-byte aligned),
// one 16-byte load per fp32 register or per two bf16 registers
__device__ __forceinline__ void load_wr(floatx4* dst, const float* p, int count) {
    for (int q = 0; q < count; ++q) dst[q] = *reinterpret_cast<const floatx4*>(p + 4 * q);
}
__device__ __forceinline__ void load_wr(u32x2* dst, const bf16_t* p, int count) {
    int q = 0;
    for (; q + 1 < count; q += 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p + 4 * q);
        dst[q] = u32x2{v[0], v[1]};
        dst[q + 1] = u32x2{v[2], v[3]};
    }
    if (q < count) dst[q] = *reinterpret_cast<const u32x2*>(p + 4 * q);
}
__device__ __forceinline__ float w_at(const floatx4& r, int k) { return r[k]; }
__device__ __forceinline__ float w_at(const u32x2& r, int k) { return (k & 1) ? bf16_hi(r[k >> 1]) : bf16_lo(r[k >> 1]); }

// Four consecutive stage values of X widened to fp32 (from LDS).
__device__ __forceinline__ floatx4 lds_x4(const unsigned char* p, float) {
    return *reinterpret_cast<const floatx4*>(p);
}
__device__ __forceinline__ floatx4 lds_x4(const unsigned char* p, bf16_t) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return floatx4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}

template <int M, int N, int NW, typename TX, typename TW>
__global__ __launch_bounds__(NW * 64 + (NW == 16 ? 0 : 64)) void monarch_pair_kernel(const TX* __restrict__ X,
                                                                const TW* KF,
                                                                const TW* KG,
                                                                float* __restrict__ Y, MonArgs args) {
    using S = MonShape<M, N, NW>;
    constexpr int kConsumerThreads = S::CONSUMERS;
    extern __shared__ __align__(16) unsigned char lds[];
    const int t = threadIdx.x;
    const int64_t row_begin = int64_t(blockIdx.x) * args.rows_per_split;
    if (row_begin >= args.batch) return;
    const int64_t row_end = min(args.batch, row_begin + int64_t(args.rows_per_split));
    const int nsteps = static_cast<int>((row_end - row_begin + kR - 1) / kR);
    auto stage = [&](int s) { return reinterpret_cast<float*>(lds + (s % S::STAGES) * S::STAGE_BYTES); };

    // instruction i of a stage's copy fills LDS vectors [64 i, 64 i + 64):
    // row r, index x, vector v of the row's x-th run of N values (N / 4 fp32
    // or N / 8 bf16 vectors); padding vectors (and any past the stage) load
    // the stage's first vector
    constexpr int EB = sizeof(TX);
    auto x_offset = [&](int i, int lane) -> uint32_t {
        constexpr int XIN = N * EB / 16;
        const int q = 64 * i + lane;
        const int r = q / (S::RP / 4), u = q - r * (S::RP / 4);
        const int x = u / (S::XP / 4), v = u - x * (S::XP / 4);
        return (r < kR && x < M && v < XIN) ? static_cast<uint32_t>((r * args.n + x * N) * EB + 16 * v) : 0u;
    };
    if (!S::SELF && t >= kConsumerThreads) {
        // ------------------------------------------------------ loader wave
        const int lane = t - kConsumerThreads;
        uint32_t off[S::INSTS];
#pragma unroll
        for (int i = 0; i < S::INSTS; ++i) off[i] = x_offset(i, lane);
        auto issue = [&](int s) {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const uint32_t limit = stage_limit(n0, row_end, args.n, EB);
            const char* base = reinterpret_cast<const char*>(X + n0 * args.n);
            unsigned char* st = reinterpret_cast<unsigned char*>(stage(s));
#pragma unroll
            for (int i = 0; i < S::INSTS; ++i)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (off[i] < limit ? off[i] : 0u)),
                                                 st + 1024 * i, 16, 0, 0);
        };
        for (int s = 0; s < S::STAGES && s < nsteps; ++s) issue(s);
        for (int s = 0; s < nsteps; ++s) {
            // stage s has landed once only the stages issued after it remain
            // (a count above vmcnt's 63 waits a little longer, never less)
            wait_vmcnt_upto(min(63, min(S::STAGES - 1, nsteps - 1 - s) * S::INSTS));
            lds_barrier();                                   // stage s ready
            lds_barrier();                                   // Z written
            lds_barrier();                                   // Y written
            lds_barrier();                                   // stage s read out
            if (s + S::STAGES < nsteps) issue(s + S::STAGES);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    // v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + i][l % 16] in register i.
    // Lane group g = l / 16 takes k = (K / 4) g + ks in step ks.
    //
    // The weights of a wave's groups are the same for every stage, so they
    // are loaded once and stay in registers. A chunk is one group's B
    // operands for this lane: F block j (CF 4-value registers) or G position
    // p (CG): (M N N + N M M) / (64 NW) registers a lane, at most 96 with
    // four waves, 64 with sixteen for M = N = 32. bf16 weights stay packed
    // and widen at use.
    using WR = typename WReg<TW>::type;
    constexpr int CF = S::NTF * (S::KSF / 4);
    constexpr int CG = S::NTG * (S::KSG / 4);
    constexpr int kChunks = S::GA + S::GB;
    constexpr int kRegs = S::GA * CF + S::GB * CG;
    static_assert(kRegs * sizeof(WR) / 4 <= 96, "weights a lane");

    const int w = t >> 6;
    const int lane = t & 63;
    const int col = lane & 15;
    const int g = lane >> 4;

    WR wr[kRegs];
    // where chunk c (0 <= c < kChunks) lives in wr
    auto chunk_base = [&](int c) constexpr { return c < S::GA ? c * CF : S::GA * CF + (c - S::GA) * CG; };
    // load chunk c into its registers. Addresses are a wave-uniform base
    // (scalar registers) plus this lane's 32-bit byte offset, which keeps
    // per-chunk addresses out of VGPRs.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const char* kf = reinterpret_cast<const char*>(KF + int64_t(wu) * S::GA * N * N);
    const char* kg = reinterpret_cast<const char*>(KG + int64_t(wu) * S::GB * M * M);
    const uint32_t lf = static_cast<uint32_t>((col * N + S::KSF * g) * sizeof(TW));
    const uint32_t lg = static_cast<uint32_t>((col * M + S::KSG * g) * sizeof(TW));
    auto load_chunk = [&](int c) {
        const int base = chunk_base(c);
        if (c < S::GA) {
            // K_F[alpha = w GA + c][0][beta = 16 nt + col][gamma = KSF g ..]
#pragma unroll
            for (int nt = 0; nt < S::NTF; ++nt)
                load_wr(wr + base + nt * (S::KSF / 4),
                        reinterpret_cast<const TW*>(kf + (c * N + 16 * nt) * N * sizeof(TW) + lf), S::KSF / 4);
        } else {
            // K_G[0][beta = w GB + p][beta' = 16 nt + col][alpha = KSG g ..]
            const int p = c - S::GA;
#pragma unroll
            for (int nt = 0; nt < S::NTG; ++nt)
                load_wr(wr + base + nt * (S::KSG / 4),
                        reinterpret_cast<const TW*>(kg + (p * M + 16 * nt) * M * sizeof(TW) + lg), S::KSG / 4);
        }
    };
#pragma unroll
    for (int c = 0; c < kChunks; ++c) load_chunk(c);

    // SELF: every wave copies instructions w, w + NW, .. of each stage with
    // LDS DMA issued from inline assembly (the compiler would wait for any
    // LDS DMA in flight before each LDS read, serialising the next stage's
    // copy with this stage's products). The weights are waited for here,
    // once: the compiler, unaware of the copies, would otherwise wait for
    // every request in flight at their first use inside the stage loop.
    constexpr int kOwnMax = (S::INSTS + NW - 1) / NW;
    const int own = (S::INSTS - w + NW - 1) / NW;            // this wave's instructions a stage
    uint32_t soff[kOwnMax];
    auto self_issue = [&](int s) {
        const int64_t n0 = row_begin + int64_t(s) * kR;
        const uint32_t limit = stage_limit(n0, row_end, args.n, EB);
        const char* base = reinterpret_cast<const char*>(X + n0 * args.n);
        const uint32_t st0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) +
                             static_cast<uint32_t>((s % S::STAGES) * S::STAGE_BYTES);
#pragma unroll
        for (int m = 0; m < kOwnMax; ++m) {
            const int i = wu + NW * m;
            if (i < S::INSTS) {
                const void* g = base + (soff[m] < limit ? soff[m] : 0u);
                asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                             "s"(st0 + 1024u * i)
                             : "memory");
            }
        }
    };
    if constexpr (S::SELF) {
#pragma unroll
        for (int m = 0; m < kOwnMax; ++m) soff[m] = x_offset(w + NW * m, lane);
        wait_vmcnt<0>();
        self_issue(0);
        if (nsteps > 1) self_issue(1);
    }
    (void)own;
    (void)soff;

    // this lane's X values of F block alpha: X[col][alpha][KSF g ..]
    auto read_x = [&](const float* st, int alpha, floatx4 (&xv)[S::KSF / 4]) {
        const unsigned char* xr =
            reinterpret_cast<const unsigned char*>(st + col * S::RP + alpha * S::XP) + S::KSF * g * sizeof(TX);
#pragma unroll
        for (int q = 0; q < S::KSF / 4; ++q) xv[q] = lds_x4(xr + 4 * q * sizeof(TX), TX());
    };
    // Z[col][alpha = KSG g + ks][beta0 .. beta0 + BB - 1]
    using ZV = typename std::conditional<S::BB == 4, floatx4, floatx2>::type;
    auto read_z = [&](const float* st, int ks, int beta0) {
        return *reinterpret_cast<const ZV*>(st + col * S::RP + (S::KSG * g + ks) * S::XP + beta0);
    };

    for (int s = 0; s < nsteps; ++s) {
        float* st = stage(s);
        if constexpr (S::SELF) {
            // this wave's part of stage s has landed once only what it issued
            // after it remains: stage s - 1's stores and stage s + 1's copy
            constexpr int kStores = kR * M * S::XVEC / kConsumerThreads;
            wait_vmcnt_upto((s >= 1 ? kStores : 0) + (s + 1 < nsteps ? own : 0));
        }
        lds_barrier();                                                   // stage s ready
        // (A) Z[r][alpha][beta] = sum_gamma K_F[alpha][0][beta][gamma] X[r][alpha][gamma].
        // Block j + 1's inputs are read before block j's results are
        // written (other slots of the row, so the order is free).
        floatx4 xn[S::KSF / 4];
        read_x(st, w * S::GA, xn);
#pragma unroll
        for (int j = 0; j < S::GA; ++j) {
            const int alpha = w * S::GA + j;
            floatx4 xv[S::KSF / 4];
#pragma unroll
            for (int q = 0; q < S::KSF / 4; ++q) xv[q] = xn[q];
            if (j + 1 < S::GA) read_x(st, alpha + 1, xn);
            const int base = chunk_base(j);
            floatx4 acc[S::NTF];
#pragma unroll
            for (int nt = 0; nt < S::NTF; ++nt) acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < S::KSF; ++ks)
#pragma unroll
                for (int nt = 0; nt < S::NTF; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        xv[ks / 4][ks % 4], w_at(wr[base + nt * (S::KSF / 4) + ks / 4], ks % 4), acc[nt], 0, 0, 0);
#pragma unroll
            for (int nt = 0; nt < S::NTF; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[(4 * g + i) * S::RP + alpha * S::XP + 16 * nt + col] = acc[nt][i];
        }
        lds_barrier();                                                   // Z written
        // (B) Y[r][beta'][beta] = sum_alpha K_G[0][beta][beta'][alpha] Z[r][alpha][beta], BB beta at a time
#pragma unroll
        for (int j = 0; j < S::GB; j += S::BB) {
            const int beta0 = w * S::GB + j;
            floatx4 acc[S::BB][S::NTG];
#pragma unroll
            for (int u = 0; u < S::BB; ++u)
#pragma unroll
                for (int nt = 0; nt < S::NTG; ++nt) acc[u][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < S::KSG; ++ks) {
                const ZV zv = read_z(st, ks, beta0);
#pragma unroll
                for (int u = 0; u < S::BB; ++u) {
                    const int base = chunk_base(S::GA + j + u);
#pragma unroll
                    for (int nt = 0; nt < S::NTG; ++nt)
                        acc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            zv[u], w_at(wr[base + nt * (S::KSG / 4) + ks / 4], ks % 4), acc[u][nt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int nt = 0; nt < S::NTG; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* zp = st + (4 * g + i) * S::RP + (16 * nt + col) * S::XP + beta0;
                    if constexpr (S::BB == 4)
                        *reinterpret_cast<floatx4*>(zp) = floatx4{acc[0][nt][i], acc[1][nt][i], acc[2][nt][i], acc[3][nt][i]};
                    else
                        *reinterpret_cast<floatx2*>(zp) = floatx2{acc[0][nt][i], acc[1][nt][i]};
                }
        }
        lds_barrier();                                                   // Y written
        // (C) the rows out: thread t takes 16-byte vectors t, t + 256, .. of
        // the stage's rows in Y's order, in two halves (half the registers)
        {
            const int64_t n0 = row_begin + int64_t(s) * kR;
            const int rows = static_cast<int>(min(int64_t(kR), row_end - n0));
            constexpr int VPR = M * S::XVEC;                 // vectors per row of Y
            constexpr int PER = kR * VPR / kConsumerThreads; // vectors per thread
            static_assert(PER % 2 == 0, "halves");
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                floatx4 v[PER / 2];
#pragma unroll
                for (int j = 0; j < PER / 2; ++j) {
                    const int q = t + kConsumerThreads * (h * (PER / 2) + j);
                    const int r = q / VPR, u = q - r * VPR, x = u / S::XVEC, e = u - x * S::XVEC;
                    v[j] = *reinterpret_cast<const floatx4*>(st + r * S::RP + x * S::XP + 4 * e);
                }
#pragma unroll
                for (int j = 0; j < PER / 2; ++j) {
                    const int q = t + kConsumerThreads * (h * (PER / 2) + j);
                    const int r = q / VPR, u = q - r * VPR;
                    if (r < rows)
                        __builtin_nontemporal_store(v[j], reinterpret_cast<floatx4*>(Y + (n0 + r) * args.n + 4 * u));
                }
            }
            lds_barrier();                                               // stage s read out
        }
        if constexpr (S::SELF) {
            if (s + S::STAGES < nsteps) self_issue(s + S::STAGES);
        }
    }
    // the ring's last prefetches (of a stage that does not come) land
    // before the wave ends
    wait_vmcnt<0>();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int M, int N, int NW, typename TX, typename TW>
ks_status_t launch_mn(const void* W0, const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                      int num_cus) {
    using S = MonShape<M, N, NW>;
    MonArgs args;
    args.n = int64_t(M) * N;
    args.batch = batch;
    // one workgroup per compute unit, equal row shares
    const int64_t steps_total = (batch + kR - 1) / kR;
    const int64_t per_cu = std::max<int64_t>(1, (160 * 1024) / (int64_t(S::STAGES) * S::STAGE_BYTES));
    const int64_t wgs = std::max<int64_t>(1, int64_t(std::max(num_cus, 1)) * per_cu);
    const int64_t steps = std::max<int64_t>(1, (steps_total + wgs - 1) / wgs);
    args.rows_per_split = static_cast<int>(steps * kR);
    const int64_t blocks = (batch + args.rows_per_split - 1) / args.rows_per_split;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    return launch_kernel(monarch_pair_kernel<M, N, NW, TX, TW>, dim3(static_cast<unsigned>(blocks)), dim3(S::THREADS),
                         size_t(S::STAGES) * S::STAGE_BYTES, stream, static_cast<const TX*>(X),
                         static_cast<const TW*>(W0), static_cast<const TW*>(W1), Y, args);
}

template <typename TX, typename TW>
ks_status_t launch_typed(int M, int N, const void* W0, const void* W1, const void* X, float* Y, int64_t batch,
                         hipStream_t stream, int num_cus) {
    // 32 x 32 blocks take sixteen compute waves, which hold all of the
    // pair's weights in registers (65,536 rows, fp32: 115 us; streaming them
    // from L2 for each stage through register rings of eight waves took 182)
    if (M == 16 && N == 16) return launch_mn<16, 16, 4, TX, TW>(W0, W1, X, Y, batch, stream, num_cus);
    if (M == 16 && N == 32) return launch_mn<16, 32, 4, TX, TW>(W0, W1, X, Y, batch, stream, num_cus);
    if (M == 32 && N == 16) return launch_mn<32, 16, 4, TX, TW>(W0, W1, X, Y, batch, stream, num_cus);
    if (M == 32 && N == 32) return launch_mn<32, 32, 16, TX, TW>(W0, W1, X, Y, batch, stream, num_cus);
    return KS_ERR_UNSUPPORTED;
}

}  // namespace

bool monarch_pair_supports(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1) {
    // fp32 X with fp32 or bf16 weights, or bf16 X with bf16 weights
    if (wt0 != wt1 || !(wt0 == kF32 || wt0 == kBF16) || !(xt == kF32 || xt == wt0)) return false;
    const int M = s0.a, N = s0.b;
    if (!((M == 16 || M == 32) && (N == 16 || N == 32))) return false;
    return s0.c == N && s0.d == 1 && s1.a == 1 && s1.b == M && s1.c == M && s1.d == N;
}

bool monarch_pair_aligned(const void* X, const void* Y) { return aligned16(X) && aligned16(Y); }

ks_status_t launch_monarch_pair(const Shape& s0, const Shape& s1, int xt, int wt0, int wt1, const void* W0,
                                const void* W1, const void* X, float* Y, int64_t batch, hipStream_t stream,
                                int num_cus) {
    if (!monarch_pair_supports(s0, s1, xt, wt0, wt1) || !monarch_pair_aligned(X, Y)) return KS_ERR_UNSUPPORTED;
    if (wt0 == kF32) return launch_typed<float, float>(s0.a, s0.b, W0, W1, X, Y, batch, stream, num_cus);
    if (xt == kF32) return launch_typed<float, bf16_t>(s0.a, s0.b, W0, W1, X, Y, batch, stream, num_cus);
    return launch_typed<bf16_t, bf16_t>(s0.a, s0.b, W0, W1, X, Y, batch, stream, num_cus);
}

}  // namespace ks
