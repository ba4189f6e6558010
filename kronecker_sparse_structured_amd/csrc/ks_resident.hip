// ks_resident.hip -- a radix-2 or radix-4 butterfly run in one persistent
// launch, with all of its weights held in registers.
//
// Butterfly layers are chains of KS factors (KS abstract page, taxoreview.com
// "dblp:303/4794", first paragraph, first sentence). A radix-2 or radix-4
// butterfly on rows of n = 4^m values (m = 4, 5, 6) is a run of factors
// (a, b, b, d), b in {2, 4}, each mixing one b-ary digit of the row index
// (bits [log2 d, log2 d + log2 b)) with a b x b block K[alpha][delta] chosen
// by the other bits. Its weights total n b log_b(n) values: 384 KB of fp32
// for n = 4096, which fits in one compute unit's 512 KB register file. So
// one workgroup of 1024 threads a compute unit keeps every block it needs in
// registers for the whole launch and streams blocks of rows through LDS;
// nothing about the weights is read per row block.
//
// Passes. The run is cut into passes that each mix one aligned 2-bit digit
// (index bits p, p + 1; p even): one radix-4 factor, or two consecutive
// radix-2 factors on bits p and p + 1 (either order). In a pass a thread
// holds the 4 values of a row that differ only in that digit (its "column")
// with its column's 16 weights, so a pass is 16 FMAs per column and row and
// six passes (n = 4096) keep 96 weights a thread.
//
// Columns and LDS banks. Rows sit in LDS in natural order. In a pass the 64
// lanes of a wave take 64 columns chosen so that, at every one of the four
// reads and writes, they hit 64 distinct banks (32 distinct in each half):
// for p >= 6 the lanes vary index bits 0..5; for p = 4 bits 0..3 and 6..7;
// for p = 2 bits 0..1, 4..5 and 6..7; the waves vary the remaining bits,
// and what is left over selects rows (n < 4096). Where the digit lies in
// the bank bits (p = 2, 4) lane l handles its values in the order e ^ r, r
// = its column's bits 6..7, so that the lanes of one read spread over the
// four digit values; its weights are stored permuted to match. For p = 0 a
// thread's four values are consecutive: one 16-byte access.
//
// Pipeline. Each workgroup takes row blocks blockIdx.x, + gridDim.x, ...
// (64 KB of fp32 rows each; 4, 16 or 64 rows). Every wave copies its share
// of block i + 1 from HBM into the other LDS buffer with LDS DMA
// (global_load_lds_dwordx4, 1 KB an instruction) while block i is computed;
// bf16 X lands in a bf16 staging buffer and the first pass widens it. The
// last pass stores Y straight from registers (16-byte stores for p = 0,
// 256-byte wave-wide runs for p >= 6). The DMA is issued from inline
// assembly: the compiler would otherwise wait for every LDS DMA in flight
// before any LDS read, which would serialise block i + 1's copy with block
// i's passes. The asm has no register outputs; completion is an explicit
// vmcnt wait (the wave's stores of the previous block are the only vector
// memory operations issued after the DMA, and their count is known) followed
// by an LDS barrier.

#include <algorithm>
#include <cstdio>

#include "ks_device.h"
#include "ks_internal.h"
#include "ks_stream.h"

namespace ks {
namespace {

constexpr int kThreads = 1024;           // 16 waves: four a SIMD, 128 VGPRs each
constexpr int kMaxPasses = 6;            // n <= 4096
constexpr int kMaxRun = 2 * kMaxPasses;
constexpr int kRowsPerThread = 4;
constexpr int kBlockBytes = 64 * 1024;   // one block of fp32 rows
constexpr int kRowStride = 16 * 1024;    // LDS bytes between a thread's rows
constexpr int kLdsBytes = 2 * kBlockBytes;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t uint32x2 __attribute__((ext_vector_type(2)));

// Pass kinds: one radix-4 factor; two radix-2 factors, bit p first; two
// radix-2 factors, bit p + 1 first.
enum PassKind : int { kRadix4 = 0, kLowFirst = 1, kHighFirst = 2 };

struct ResArgs {
    int lg;                          // log2 of the row width (of a slab)
    int npass;
    int rows;                        // rows per block
    int nblocks;                     // row blocks (of each slab)
    int64_t batch;
    int slabs;                       // slabs of a row, each its own butterfly; workgroups take one each
    int64_t ldx, ldy;                // elements from one row of X / Y to the next
    const void* w0[kMaxPasses];      // the pass's (first) factor
    const void* w1[kMaxPasses];      // its second radix-2 factor
    int64_t ws0[kMaxPasses];         // elements of w0 / w1 from one slab's blocks to the next
    int64_t ws1[kMaxPasses];
};

// The column of thread t in a pass on digit bits p, p + 1 of an L-bit index:
// its free bits (base), the rotation r of its digit order, and its row group.
__device__ __forceinline__ void column_of(int p, int L, int t, int& base, int& r, int& g) {
    const int l = t & 63;
    int lane_bits, used;
    if (p >= 6) {
        lane_bits = l;
        used = 63;
        r = 0;
    } else if (p == 4) {
        lane_bits = (l & 15) | ((l >> 4) << 6);
        used = 15 | (3 << 6);
        r = l >> 4;
    } else if (p == 2) {
        lane_bits = (l & 3) | (((l >> 4) & 3) << 4) | (((l >> 2) & 3) << 6);
        used = 3 | (3 << 4) | (3 << 6);
        r = (l >> 2) & 3;
    } else {
        lane_bits = l << 2;
        used = 63 << 2;
        r = 0;
    }
    const int free = ((1 << L) - 1) & ~(3 << p) & ~used;
    int w = t >> 6, out = lane_bits;
    for (int bit = 0; bit < L; ++bit) {
        if ((free >> bit) & 1) {
            out |= (w & 1) << bit;
            w >>= 1;
        }
    }
    base = out;
    g = w;
}

// The 16 weights of a thread's column for one pass, in the order the pass
// applies them (register e holds the value of digit e ^ r).
template <typename TW>
__device__ __forceinline__ void load_pass_weights(float (&w)[16], const TW* K0, const TW* K1, int kind, int p,
                                                  int base, int r) {
    if (kind == kRadix4) {
        // block (alpha, delta) of the factor (a, 4, 4, 2^p): alpha above the digit, delta below
        const int64_t blk = (int64_t(base >> (p + 2)) << p) + (base & ((1 << p) - 1));
        const TW* k = K0 + blk * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) w[e * 4 + e2] = to_f32(k[((e ^ r) << 2) | (e2 ^ r)]);
        return;
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        // factor f acts on register bit jb, i.e. index bit q = p + jb
        const int jb = (kind == kLowFirst) ? f : 1 - f;
        const int q = p + jb;
        const int s = (r >> jb) & 1;
        const TW* K = f == 0 ? K0 : K1;
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int e0 = o << (1 - jb);                   // register with bit jb clear, other bit o
            const int idx = base + ((e0 ^ r) << p);         // its index in the row
            const int64_t blk = (int64_t(idx >> (q + 1)) << q) + (idx & ((1 << q) - 1));
            const TW* k = K + blk * 4;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) w[f * 8 + o * 4 + b * 2 + b2] = to_f32(k[((b ^ s) << 1) | (b2 ^ s)]);
        }
    }
}

__device__ __forceinline__ void pair(float& x0, float& x1, const float* w) {
    const float y0 = fmaf(w[1], x1, fmaf(w[0], x0, 0.0f));
    const float y1 = fmaf(w[3], x1, fmaf(w[2], x0, 0.0f));
    x0 = y0;
    x1 = y1;
}

__device__ __forceinline__ void apply(float (&v)[4], const float (&w)[16], int kind) {
    if (kind == kRadix4) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) acc = fmaf(w[e * 4 + e2], v[e2], acc);
            y[e] = acc;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = y[e];
    } else if (kind == kLowFirst) {
        pair(v[0], v[1], w + 0);
        pair(v[2], v[3], w + 4);
        pair(v[0], v[2], w + 8);
        pair(v[1], v[3], w + 12);
    } else {
        pair(v[0], v[2], w + 0);
        pair(v[1], v[3], w + 4);
        pair(v[0], v[1], w + 8);
        pair(v[2], v[3], w + 12);
    }
}

// One 1 KB LDS DMA: lane l's 16 bytes at g land at LDS byte lds + 16 l.
__device__ __forceinline__ void dma_1k(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}

// Copy block `blk` of X (X points at the workgroup's slab of row 0) into
// LDS at byte `dst`, rows packed: each wave its share of 1 KB chunks, chunk
// c being 1 KB (c mod chunks-per-row) of row c / chunks-per-row. Returns
// nothing; the wave's vmcnt covers its chunks.
template <typename TX>
__device__ __forceinline__ void issue_block(const TX* X, const ResArgs& a, int blk, uint32_t dst) {
    const int64_t row0 = int64_t(blk) * a.rows;
    const int nr = static_cast<int>(min(int64_t(a.rows), a.batch - row0));
    const int row_log = a.lg + (sizeof(TX) == 2 ? 1 : 2) - 10;      // log2 of 1 KB chunks a row (>= 1)
    const int chunks = nr << row_log;
    const int64_t ld_bytes = a.ldx * int64_t(sizeof(TX));
    constexpr int per_wave = (kBlockBytes * sizeof(TX) / 4) / 1024 / (kThreads / 64);
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const char* src = reinterpret_cast<const char*>(X) + row0 * ld_bytes + (threadIdx.x & 63) * 16;
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
        const int c = w * per_wave + j;
        if (c < chunks) {
            const int r = c >> row_log;
            const int part = c - (r << row_log);
            dma_1k(src + int64_t(r) * ld_bytes + part * 1024, dst + c * 1024);
        }
    }
}

// The chain's shape is compile-time: rows of 2^L values, radix B, digits
// descending (d = n / B first) or ascending along the run; pass ps mixes
// index bits p(ps), p(ps) + 1.
template <int L, int B, int DESC>
struct Chain {
    static constexpr int NP = L / 2;
    static constexpr int kind = B == 4 ? kRadix4 : (DESC ? kHighFirst : kLowFirst);
    static constexpr int p(int ps) { return DESC ? L - 2 - 2 * ps : 2 * ps; }
    static constexpr int Q = 1 << (12 - L);          // row groups
};

// Wait until at most n of this wave's vector-memory operations are in
// flight, n being a count of one block's stores: 0..4 (16-byte stores) or a
// multiple of 4 up to 16 (4-byte stores).
__device__ __forceinline__ void wait_stores(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 12: wait_vmcnt<12>(); break;
        default: wait_vmcnt<16>(); break;
    }
}

template <typename TX, typename TW, int L, int B, int DESC>
__global__ __launch_bounds__(kThreads) void resident_chain_kernel(const TX* __restrict__ X, float* __restrict__ Y,
                                                                  ResArgs args) {
    using C = Chain<L, B, DESC>;
    constexpr bool kWiden = sizeof(TX) == 2;
    extern __shared__ __align__(16) unsigned char lds[];
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
    const int t = threadIdx.x;
    // fp32: the DMA fills work buffer (i & 1) and the passes run in it;
    // bf16: the DMA fills staging buffer (i & 1) and the first pass writes work buffer 0
    auto dma_dst = [&](int b) -> uint32_t {
        return lds0 + (kWiden ? kBlockBytes + b * (kBlockBytes / 2) : b * kBlockBytes);
    };

    // workgroup: slab blockIdx.x % slabs (its weights), row blocks
    // blockIdx.x / slabs, + gridDim.x / slabs, ... (the grid is a multiple of
    // the slab count)
    const int slab = static_cast<int>(blockIdx.x % static_cast<unsigned>(args.slabs));
    const int bstep = static_cast<int>(gridDim.x / static_cast<unsigned>(args.slabs));
    X += int64_t(slab) << L;
    Y += int64_t(slab) << L;
    int bi = static_cast<int>(blockIdx.x / static_cast<unsigned>(args.slabs));
    if (bi < args.nblocks) issue_block(X, args, bi, dma_dst(0));

    float wr[C::NP][16];
    int addr[C::NP];                             // LDS byte offset of value 0 of the thread's first row
    int g = 0, base_last = 0;
#pragma unroll
    for (int ps = 0; ps < C::NP; ++ps) {
        const int p = C::p(ps);
        int base, r;
        column_of(p, L, t, base, r, g);
        addr[ps] = ((base | (r << p)) << 2) + (g << (L + 2));
        if (ps == C::NP - 1) base_last = base;
        const TW* k0 = static_cast<const TW*>(args.w0[ps]) + slab * args.ws0[ps];
        const TW* k1 = args.w1[ps] ? static_cast<const TW*>(args.w1[ps]) + slab * args.ws1[ps] : nullptr;
        load_pass_weights<TW>(wr[ps], k0, k1, C::kind, p, base, r);
    }
    const int gq = __builtin_amdgcn_readfirstlane(g);

    int nst = 0;                                 // this wave's stores of the previous block
    for (int it = 0; bi < args.nblocks; bi += bstep, ++it) {
        const int cur = it & 1;
        wait_stores(nst);                        // this wave's chunks of block bi have landed
        lds_barrier();                           // every wave's have; the previous block is done
        if (bi + bstep < args.nblocks) issue_block(X, args, bi + bstep, dma_dst(cur ^ 1));
        const int64_t row0 = int64_t(bi) * args.rows;
        const int nr = static_cast<int>(min(int64_t(args.rows), args.batch - row0));
        const uint32_t work = kWiden ? 0u : static_cast<uint32_t>(cur * kBlockBytes);
        const uint32_t stage = dma_dst(cur) - lds0;
        nst = 0;
#pragma unroll
        for (int ps = 0; ps < C::NP; ++ps) {
            constexpr int kind = C::kind;
            const int p = C::p(ps);
            const bool last = ps == C::NP - 1;
            if (ps > 0) lds_barrier();
            // rows interleaved for LDS latency: all four (fp32 X), two at a
            // time where widening bf16 X needs the registers
            constexpr int kInterleave = kWiden ? 2 : kRowsPerThread;
#pragma unroll kInterleave
            for (int j = 0; j < kRowsPerThread; ++j) {
                float v[4];
                if (kWiden && ps == 0) {
                    const uint32_t sa = stage + (addr[ps] >> 1) + j * (kRowStride / 2);
                    if (p == 0) {
                        const uint32x2 u = *static_cast<const uint32x2*>(__builtin_assume_aligned(lds + sa, 8));
                        v[0] = bf16_lo(u[0]);
                        v[1] = bf16_hi(u[0]);
                        v[2] = bf16_lo(u[1]);
                        v[3] = bf16_hi(u[1]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = to_f32(*reinterpret_cast<const bf16_t*>(lds + (sa ^ (e << (p + 1)))));
                    }
                } else {
                    const uint32_t wa = work + addr[ps] + j * kRowStride;
                    if (p == 0) {
                        const floatx4 x = *static_cast<const floatx4*>(__builtin_assume_aligned(lds + wa, 16));
                        v[0] = x[0];
                        v[1] = x[1];
                        v[2] = x[2];
                        v[3] = x[3];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const float*>(lds + (wa ^ (e << (p + 2))));
                    }
                }
                apply(v, wr[ps], kind);
                if (!last) {
                    const uint32_t wa = work + addr[ps] + j * kRowStride;
                    if (p == 0) {
                        *static_cast<floatx4*>(__builtin_assume_aligned(lds + wa, 16)) = floatx4{v[0], v[1], v[2], v[3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) *reinterpret_cast<float*>(lds + (wa ^ (e << (p + 2)))) = v[e];
                    }
                } else if (gq + C::Q * j < nr) {
                    float* yr = Y + (row0 + gq + C::Q * j) * args.ldy;
                    if (p == 0) {
                        __builtin_nontemporal_store(floatx4{v[0], v[1], v[2], v[3]},
                                                    reinterpret_cast<floatx4*>(yr + base_last));
                        nst += 1;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) __builtin_nontemporal_store(v[e], yr + (base_last ^ (e << p)));
                        nst += 4;
                    }
                }
            }
        }
    }
}

int log2i(int64_t v) {
    int l = 0;
    while ((int64_t(1) << l) < v) ++l;
    return l;
}

// The run as a whole butterfly on 2^lg-wide rows: every factor (a, b, b, d)
// of one radix b in {2, 4}, digits covering the index bits once each, in
// descending (d = n / b first) or ascending order. False if it is not one.
struct Form {
    int lg, radix, desc;
};
bool form_of(const Shape* s, int n, int slabs, Form* f) {
    if (n < 2 || n > kMaxRun || slabs < 1) return false;
    if (s[0].n_in % slabs != 0) return false;
    const int64_t w = s[0].n_in / slabs;         // each slab's width
    if (!(w == 1024 || w == 4096)) return false;
    const int b = s[0].b;
    if (!(b == 2 || b == 4)) return false;
    f->lg = log2i(w);
    f->radix = b;
    const int q = log2i(b);
    if (n * q != f->lg) return false;
    f->desc = s[0].d > s[1].d ? 1 : 0;
    for (int k = 0; k < n; ++k) {
        if (s[k].a % slabs != 0) return false;
        if (s[k].b != b || s[k].c != b || s[k].n_in != w * slabs || s[k].n_out != w * slabs) return false;
        const int64_t d = int64_t(1) << (f->desc ? f->lg - q * (k + 1) : q * k);
        if (s[k].d != d || int64_t(s[k].a / slabs) * b * d != w) return false;
    }
    return true;
}

template <typename TX, typename TW, int L>
ks_status_t launch_shape(const ResArgs& a, int grid, int radix, int desc, const void* X, float* Y,
                         hipStream_t stream) {
    const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
    const TX* x = static_cast<const TX*>(X);
    if (radix == 4 && desc) return launch_kernel(resident_chain_kernel<TX, TW, L, 4, 1>, g, blk, kLdsBytes, stream, x, Y, a);
    if (radix == 4) return launch_kernel(resident_chain_kernel<TX, TW, L, 4, 0>, g, blk, kLdsBytes, stream, x, Y, a);
    if (desc) return launch_kernel(resident_chain_kernel<TX, TW, L, 2, 1>, g, blk, kLdsBytes, stream, x, Y, a);
    return launch_kernel(resident_chain_kernel<TX, TW, L, 2, 0>, g, blk, kLdsBytes, stream, x, Y, a);
}

template <typename TX, typename TW>
ks_status_t launch_typed(const ResArgs& a, int grid, int radix, int desc, const void* X, float* Y,
                         hipStream_t stream) {
    if (a.lg == 12) return launch_shape<TX, TW, 12>(a, grid, radix, desc, X, Y, stream);
    return launch_shape<TX, TW, 10>(a, grid, radix, desc, X, Y, stream);
}

}  // namespace

bool resident_types(int xt, int wt) {
    return (xt == kF32 || xt == kBF16) && (wt == kF32 || wt == kBF16) && !(xt == kBF16 && wt == kF32);
}

bool resident_chain_supports(const Shape* s, int n, int xt, int wt) {
    Form f{};
    return form_of(s, n, 1, &f) && resident_types(xt, wt);
}

bool resident_slab_form(const Shape* s, int n, int xt, int wt, int* slabs) {
    Form f{};
    if (n < 2 || !resident_types(xt, wt)) return false;
    for (int64_t w : {int64_t(4096), int64_t(1024)}) {
        if (s[0].n_in % w != 0 || s[0].n_in / w > 0x7fffffff) continue;
        const int p = static_cast<int>(s[0].n_in / w);
        if (form_of(s, n, p, &f)) {
            *slabs = p;
            return true;
        }
    }
    return false;
}

bool resident_chain_aligned(const void* X, const float* Y) {
    return reinterpret_cast<uintptr_t>(X) % 16 == 0 && reinterpret_cast<uintptr_t>(Y) % 16 == 0;
}

ks_status_t launch_resident_slabs(const Shape* s, int n, int slabs, int xt, int wt, const void* const* W,
                                  const void* X, float* Y, int64_t batch, hipStream_t stream, int num_cus) {
    Form f{};
    if (!form_of(s, n, slabs, &f) || !resident_types(xt, wt) || !resident_chain_aligned(X, Y))
        return KS_ERR_UNSUPPORTED;
    if (batch == 0) return KS_OK;
    ResArgs a{};
    a.lg = f.lg;
    a.npass = f.lg / 2;
    for (int ps = 0; ps < a.npass; ++ps) {
        // radix 4: one factor a pass; radix 2: two, applied in run order
        const int k0 = f.radix == 4 ? ps : 2 * ps;
        a.w0[ps] = W[k0];
        a.ws0[ps] = s[k0].nnz / slabs;
        a.w1[ps] = f.radix == 4 ? nullptr : W[k0 + 1];
        a.ws1[ps] = f.radix == 4 ? 0 : s[k0 + 1].nnz / slabs;
    }
    a.rows = kBlockBytes / (4 << a.lg);
    a.batch = batch;
    a.slabs = slabs;
    a.ldx = s[0].n_in;
    a.ldy = s[n - 1].n_out;
    const int64_t blocks = (batch + a.rows - 1) / a.rows;
    if (blocks > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    a.nblocks = static_cast<int>(blocks);
    // one persistent workgroup a compute unit, the same number on every slab
    const int64_t per_slab = std::max<int64_t>(1, std::min<int64_t>(blocks, std::max(1, num_cus) / slabs));
    if (per_slab * slabs > 0x7fffffff) return KS_ERR_UNSUPPORTED;
    const int grid = static_cast<int>(per_slab * slabs);
    if (xt == kF32 && wt == kF32) return launch_typed<float, float>(a, grid, f.radix, f.desc, X, Y, stream);
    if (xt == kF32 && wt == kBF16) return launch_typed<float, bf16_t>(a, grid, f.radix, f.desc, X, Y, stream);
    return launch_typed<bf16_t, bf16_t>(a, grid, f.radix, f.desc, X, Y, stream);
}

ks_status_t launch_resident_chain(const Shape* s, int n, int xt, int wt, const void* const* W, const void* X,
                                  float* Y, int64_t batch, hipStream_t stream, int num_cus) {
    return launch_resident_slabs(s, n, 1, xt, wt, W, X, Y, batch, stream, num_cus);
}

int resident_chain_describe(const Shape* s, int n, int slabs, char* buf, size_t len) {
    Form f{};
    if (!form_of(s, n, slabs, &f)) return -1;
    char where[64] = "";
    if (slabs > 1) std::snprintf(where, sizeof(where), " on each of %d slabs of %d values", slabs, 1 << f.lg);
    std::snprintf(buf, len,
                  "register-resident butterfly%s: %d radix-%d factors in %d passes (%s), weights in registers, "
                  "rows/block=%d, lds=%d, one persistent workgroup of %d threads per CU",
                  where, n, f.radix, f.lg / 2, f.desc ? "descending" : "ascending", kBlockBytes / (4 << f.lg),
                  kLdsBytes, kThreads);
    return 0;
}

}  // namespace ks
