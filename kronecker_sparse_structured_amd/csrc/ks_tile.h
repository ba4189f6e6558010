// ks_tile.h -- the part of one row that a workgroup tile reads or writes,
// and how its 16-byte vectors map between global memory and LDS.
//
// A tile covers the alphas [alpha0, alpha0 + at) and deltas
// [delta0, delta0 + dt) of a KS factor. In a row of X (layout
// [alpha][gamma][delta]) or Y (layout [alpha][beta][delta]) that part is
//  * contiguous, when the tile spans every delta (dt == d): at slabs of
//    w*d elements each (w = c for X, b or the tile's share of b for Y),
//    slab_global elements apart; or
//  * segmented, when at == 1 and dt < d: w segments of dt elements, d apart.
// In LDS a row is stored slab after slab (contiguous) or segment after
// segment (segmented), each slab or segment padded as the kernel chooses.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace ks {

struct RowChunk {
    int contiguous;     // 1: slabs of `slab` elements; 0: `nseg` segments
    int slab;           // contiguous: elements per alpha slab in the tile
    int slab_global;    // contiguous: global elements between alpha slabs
    int lds_slab;       // contiguous: LDS bytes per slab (16-byte multiple)
    int nseg;           // segmented: segments per row (w)
    int seg_global;     // segmented: global elements between segments (d)
    int seg_lds;        // segmented: LDS bytes between segments
    int seg_cap;        // segmented: LDS elements per segment (>= dt, vw multiple)
    int lds_row;        // LDS bytes per staged row
};

// Where vector q (vw elements of eb bytes) of a row chunk lives: element
// offset in the global row chunk, byte offset in the LDS row, and whether it
// lies inside the valid part of the tile (at_eff alphas, dt_eff deltas).
__device__ __forceinline__ void chunk_vector(const RowChunk& m, int q, int vw, int at_eff,
                                             int dt_eff, int* gofs, int* lofs, bool* ok) {
    if (m.contiguous) {
        const int per = m.slab / vw;
        const int s = q / per;
        const int e = q - s * per;
        *gofs = s * m.slab_global + e * vw;
        *lofs = s * m.lds_slab + e * 16;
        *ok = s < at_eff;
    } else {
        const int per = m.seg_cap / vw;
        const int s = q / per;
        const int e = q - s * per;
        *gofs = s * m.seg_global + e * vw;
        *lofs = s * m.seg_lds + e * 16;
        *ok = s < m.nseg && e * vw < dt_eff;
    }
}

}  // namespace ks
