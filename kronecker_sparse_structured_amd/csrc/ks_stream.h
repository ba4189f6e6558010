// ks_stream.h -- streaming a workgroup's rows of X through LDS.
//
// A workgroup is kConsumers compute waves plus one loader wave. The loader
// wave moves X from HBM straight into an LDS ring of S stages with
// global_load_lds_dwordx4 (16 bytes per lane, no VGPRs), running S-1 stages
// ahead of the consumers. Only the loader wave issues loads in the streaming
// loop, so its vector-memory counter covers loads alone and "stage s has
// landed" is an exact vmcnt wait. The consumer waves read LDS, compute and
// store Y; they never wait on vector memory, so stores drain in the
// background. Hand-offs use an LDS-only barrier (no global-memory fence).
//
// Layout of one stage: R rows, each a row chunk of `blocks` blocks (alpha
// slabs or gamma segments of the tile) of blk_vec 16-byte vectors, each
// block followed by pad_vec unused vectors (to spread LDS banks), rows
// row_vec vectors apart. The loader issues exactly kStageInsts instructions
// per stage; instruction i fills LDS vectors [64 i, 64 i + 64) of the stage.
// Lanes whose vector lies in padding, beyond the tile's valid part or beyond
// the last row load a dummy vector (the first vector of the workgroup's
// first row), which nothing reads.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace ks {

constexpr int kConsumers = 4;                        // compute waves per workgroup
constexpr int kConsumerThreads = kConsumers * 64;
constexpr int kStreamThreads = kConsumerThreads + 64;

// LDS-only workgroup barrier: completes this wave's LDS operations, then
// s_barrier. Outstanding global loads and stores are not waited for.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

struct StageMap {
    int rows;          // R: rows per stage
    int blocks;        // blocks per row chunk (the tile's alpha slabs or gamma segments)
    int blk_vec;       // vectors per block
    int pad_vec;       // unused vectors after each block
    int row_vec;       // LDS pitch of a row, in vectors
    int gstride;       // global elements between consecutive blocks
};

// Wait until at most n (0..63, wave-uniform) vector-memory operations of
// this wave are in flight; s_waitcnt takes an immediate, hence the switch.
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    if constexpr (N < 63) {
        if (n == N) {
            wait_vmcnt<N>();
            return;
        }
        wait_vmcnt_upto<N + 1>(n);
    } else {
        wait_vmcnt<63>();
    }
}

// The loader lane's part of every stage: for each of its first `insts`
// (<= kMaxInsts) instructions, the byte offset of its vector from the start
// of the tile's chunk in the stage's first row (row r adds r * n_in
// elements), or kNoVector for a padding or out-of-tile position. The host
// keeps R * n_in * sizeof(element) below 2^31 so offsets fit in 32 bits.
constexpr uint32_t kNoVector = 0xffffffffu;

template <int kMaxInsts>
struct LoaderPlan {
    uint32_t off[kMaxInsts];
};

template <int kMaxInsts>
__device__ __forceinline__ void make_loader_plan(const StageMap& m, int insts, int vw, int eb, int64_t n_in,
                                                 int valid_blocks, int valid_vec, int lane,
                                                 LoaderPlan<kMaxInsts>* lp) {
    const int pitch = m.blk_vec + m.pad_vec;
#pragma unroll
    for (int i = 0; i < kMaxInsts; ++i) {
        const int p = 64 * i + lane;
        const int r = p / m.row_vec;
        const int u = p - r * m.row_vec;
        const int blk = u / pitch;
        const int e = u - blk * pitch;
        const bool ok = i < insts && r < m.rows && blk < valid_blocks && e < valid_vec;
        lp->off[i] = ok ? static_cast<uint32_t>((r * n_in + int64_t(blk) * m.gstride + int64_t(e) * vw) * eb)
                        : kNoVector;
    }
}

// Issue one stage (exactly `insts` loader instructions) into LDS at `stage`.
// `first` is the tile's chunk in the stage's first row; `limit` is
// rows_left * n_in * sizeof(element) (saturated): vectors at or beyond it
// belong to rows past the workgroup's range and load `first` instead (a
// harmless dummy nobody reads).
template <int kMaxInsts, typename T>
__device__ __forceinline__ void issue_stage(const LoaderPlan<kMaxInsts>& lp, int insts, const T* first,
                                            uint32_t limit, unsigned char* stage) {
    const char* base = reinterpret_cast<const char*>(first);
#pragma unroll
    for (int i = 0; i < kMaxInsts; ++i) {
        if (i < insts) {
            const uint32_t o = lp.off[i];
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (o < limit ? o : 0u)),
                                             stage + 1024 * i, 16, 0, 0);
        }
    }
}

// The part of a stage that loader wave `part` of `parts` issues: every
// instruction i with i % parts == part (the same addresses as issue_stage).
template <int kMaxInsts, typename T>
__device__ __forceinline__ void issue_stage_part(const LoaderPlan<kMaxInsts>& lp, int insts, const T* first,
                                                 uint32_t limit, unsigned char* stage, int part, int parts) {
    const char* base = reinterpret_cast<const char*>(first);
#pragma unroll
    for (int i = 0; i < kMaxInsts; ++i) {
        if (i < insts && i % parts == part) {
            const uint32_t o = lp.off[i];
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (o < limit ? o : 0u)),
                                             stage + 1024 * i, 16, 0, 0);
        }
    }
}

// The byte limit of issue_stage for a stage whose first row is n0.
__device__ __forceinline__ uint32_t stage_limit(int64_t n0, int64_t row_end, int64_t n_in, int eb) {
    const int64_t bytes = (row_end - n0) * n_in * eb;
    return bytes >= int64_t(kNoVector) ? kNoVector : static_cast<uint32_t>(bytes);
}

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8 picks
// the XCD). Renumber them so that consecutive logical ids run on the same
// XCD: tiles that are neighbours in the logical order (and share cache
// lines of X and Y) then share that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int block, int nblocks) {
    constexpr int kXcds = 8;
    const int per = nblocks / kXcds;            // full rounds
    const int xcd = block % kXcds;
    const int idx = block / kXcds;
    if (idx < per) return xcd * per + idx;      // the first per * 8 blocks
    return block;                               // the remainder keeps its id
}

}  // namespace ks
