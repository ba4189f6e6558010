// ks_closure.cpp -- the closure rule for fusing two consecutive KS factors.
//
// A chain of KS factors (KS abstract page, taxoreview.com "dblp:303/4794",
// first paragraph, first sentence: Butterfly and Monarch matrices are such
// chains) can run two factors F then G in one pass only if the intermediate
// Z = F(X) splits into pieces that never need each other. F computes each
// output group (fixed alpha, delta of F; all beta) from one input group
// (all gamma); G reads each input group (fixed alpha, delta of G; all gamma)
// to produce one output group. Linking the intermediate values that share
// an F output group or a G input group gives closed components: a
// component's outputs depend only on its inputs, through its own F blocks
// and G blocks. Fusion then needs, per tile of components processed
// together, the components' intermediates on chip and their weights near
// the compute units; the tile must hold enough components for its X reads
// to come in runs of at least 16 bytes.
//
// This file computes the components by union-find over the intermediate
// indices (host only, at most 2^22 of them) and reports their sizes; the
// chain planner and ks_chain_describe use it.

#include <algorithm>
#include <vector>

#include "ks_internal.h"

namespace ks {

namespace {

int find_root(std::vector<int32_t>& parent, int32_t x) {
    int32_t r = x;
    while (parent[r] != r) r = parent[r];
    while (parent[x] != r) {
        const int32_t next = parent[x];
        parent[x] = r;
        x = next;
    }
    return r;
}

void unite(std::vector<int32_t>& parent, int32_t a, int32_t b) {
    a = find_root(parent, a);
    b = find_root(parent, b);
    if (a != b) parent[std::max(a, b)] = std::min(a, b);
}

// Longest-run statistic of a sorted index set: the shortest run of
// consecutive indices in it.
int64_t shortest_run(std::vector<int64_t>& v) {
    std::sort(v.begin(), v.end());
    int64_t best = int64_t(1) << 62, run = 1;
    for (size_t i = 1; i <= v.size(); ++i) {
        if (i < v.size() && v[i] == v[i - 1] + 1) {
            ++run;
        } else {
            best = std::min(best, run);
            run = 1;
        }
    }
    return v.empty() ? 0 : best;
}

}  // namespace

bool closure_of(const Shape& f, const Shape& g, Closure* c) {
    const int64_t n_mid = f.n_out;
    if (n_mid != g.n_in || n_mid < 1 || n_mid > kMaxClosureMid) return false;
    std::vector<int32_t> parent(static_cast<size_t>(n_mid));
    for (int64_t m = 0; m < n_mid; ++m) parent[m] = static_cast<int32_t>(m);
    // F output group (alpha1, delta1): m = alpha1 b1 d1 + beta1 d1 + delta1
    for (int64_t a1 = 0; a1 < f.a; ++a1)
        for (int64_t d1 = 0; d1 < f.d; ++d1) {
            const int64_t m0 = a1 * f.b * f.d + d1;
            for (int64_t b1 = 1; b1 < f.b; ++b1)
                unite(parent, static_cast<int32_t>(m0), static_cast<int32_t>(m0 + b1 * f.d));
        }
    // G input group (alpha2, delta2): m = alpha2 c2 d2 + gamma2 d2 + delta2
    for (int64_t a2 = 0; a2 < g.a; ++a2)
        for (int64_t d2 = 0; d2 < g.d; ++d2) {
            const int64_t m0 = a2 * g.c * g.d + d2;
            for (int64_t c2 = 1; c2 < g.c; ++c2)
                unite(parent, static_cast<int32_t>(m0), static_cast<int32_t>(m0 + c2 * g.d));
        }
    std::vector<int64_t> size(static_cast<size_t>(n_mid), 0), fgroups(static_cast<size_t>(n_mid), 0),
        ggroups(static_cast<size_t>(n_mid), 0);
    for (int64_t m = 0; m < n_mid; ++m) ++size[find_root(parent, static_cast<int32_t>(m))];
    for (int64_t a1 = 0; a1 < f.a; ++a1)
        for (int64_t d1 = 0; d1 < f.d; ++d1) ++fgroups[find_root(parent, static_cast<int32_t>(a1 * f.b * f.d + d1))];
    for (int64_t a2 = 0; a2 < g.a; ++a2)
        for (int64_t d2 = 0; d2 < g.d; ++d2) ++ggroups[find_root(parent, static_cast<int32_t>(a2 * g.c * g.d + d2))];
    Closure out{};
    out.uniform = true;
    int64_t first = -1;
    for (int64_t m = 0; m < n_mid; ++m) {
        if (size[m] == 0) continue;                  // not a root
        ++out.components;
        if (first < 0) first = size[m];
        if (size[m] != first) out.uniform = false;
        if (size[m] > out.mid) {
            out.mid = size[m];
            out.inputs = fgroups[m] * f.c;
            out.outputs = ggroups[m] * g.b;
            out.weights = fgroups[m] * f.b * f.c + ggroups[m] * g.b * g.c;
        }
    }
    // runs of the component of intermediate 0 in X and in Y
    const int32_t r0 = find_root(parent, 0);
    std::vector<int64_t> xin, yout;
    for (int64_t a1 = 0; a1 < f.a; ++a1)
        for (int64_t d1 = 0; d1 < f.d; ++d1)
            if (find_root(parent, static_cast<int32_t>(a1 * f.b * f.d + d1)) == r0)
                for (int64_t c1 = 0; c1 < f.c; ++c1) xin.push_back(a1 * f.c * f.d + c1 * f.d + d1);
    for (int64_t a2 = 0; a2 < g.a; ++a2)
        for (int64_t d2 = 0; d2 < g.d; ++d2)
            if (find_root(parent, static_cast<int32_t>(a2 * g.c * g.d + d2)) == r0)
                for (int64_t b2 = 0; b2 < g.b; ++b2) yout.push_back(a2 * g.b * g.d + b2 * g.d + d2);
    out.in_run = shortest_run(xin);
    out.out_run = shortest_run(yout);
    // a tile of components whose X reads come in 16-byte runs (fp32)
    const int64_t per_tile = std::max<int64_t>(1, (4 + out.in_run - 1) / out.in_run);
    out.tile_components = std::min(per_tile, out.components);
    out.tile_weights = out.tile_components * out.weights;
    *c = out;
    return true;
}

}  // namespace ks
