"""The closure tiling of wide chains, on the CPU (no GPU needed).

A run of KS factors whose a's share a divisor P and whose d's share a
divisor Q acts independently on P contiguous slabs of a row and, within a
slab, on the Q classes of indices equal modulo Q (KS abstract page,
taxoreview.com "dblp:303/4794", first paragraph: KS factors have supports
I_a (x) 1_{b x c} (x) I_d, so a factor never mixes slabs alpha, nor indices
that differ modulo d). The tiled row-chain kernels rely on that: a tile holds
one slab's group of T classes (class fastest), and on it each factor is the
KS factor (a/P, b, c, (d/Q) T) with remapped blocks.

This test rebuilds that mapping from the rule, runs the chain tile by tile in
fp64 with numpy, and checks that every element is read and written exactly
once and that the result is the oracle chain's; and that the library's
planner reports the same tile (P, Q, T) for the run.
"""
import math
import re

import numpy as np
import pytest

import oracle
from kronecker_sparse_structured_amd import datagen, libks

MAX_WIDTH, CLASS_WIDTH, MIN_RUN, SLAB_TARGET = 4096, 1024, 32, 256


def rule_tile(pats):
    """(P, Q, T) of a run whose rows are wider than 4096 values."""
    w = max([pats[0][0] * pats[0][2] * pats[0][3]] + [p[0] * p[1] * p[3] for p in pats])
    P = Q = 0
    for a, b, c, d in pats:
        P, Q = math.gcd(P, a), math.gcd(Q, d)
    if w // P <= MAX_WIDTH:
        for f in range(1, P + 1):
            if P % f == 0 and w // f <= SLAB_TARGET:
                return f, 1, 1
        return P, 1, 1
    sub = w // (P * Q)
    for t in range(CLASS_WIDTH // sub, MIN_RUN - 1, -1):
        if Q % t == 0:
            return P, Q, t
    return None


def run_tiled(pats, X, Ws, P, Q, T):
    """The chain tile by tile: tile element e*T + t of slab p, class group q0
    is row element p*(n/P) + e*Q + q0 + t; factor (a, b, c, d) on the tile is
    (a/P, b, c, (d/Q) T) with block (alpha', delta'') taken from
    K[p a/P + alpha'][(delta''/T) Q + q0 + delta'' % T]."""
    batch, n_in = X.shape
    n_out = pats[-1][0] * pats[-1][1] * pats[-1][3]
    Y = np.full((batch, n_out), np.nan)
    reads = np.zeros(X.shape, int)
    writes = np.zeros(Y.shape, int)
    for p in range(P):
        for q0 in range(0, Q, T):
            def where(width, m):          # row positions of the tile's m values
                e, t = np.divmod(np.arange(m), T)
                return p * (width // P) + e * Q + q0 + t
            src = where(n_in, n_in // (P * Q) * T)
            reads[:, src] += 1
            z = X[:, src]
            for (a, b, c, d), K in zip(pats, Ws):
                ap, dx = a // P, d // Q * T
                out = np.empty((batch, ap * b * dx))
                for al in range(ap):
                    for de in range(dx):
                        blk = K[p * ap + al, (de // T) * Q + q0 + de % T]          # b x c
                        out[:, al * b * dx + np.arange(b) * dx + de] = z[:, al * c * dx + np.arange(c) * dx + de] @ blk.T
                z = out
            dst = where(n_out, z.shape[1])
            writes[:, dst] += 1
            Y[:, dst] = z
    assert (reads == 1).all() and (writes == 1).all()
    return Y


def _radix(r, L):
    return [(r ** k, r, r, r ** (L - 1 - k)) for k in range(L)]


RUNS = {
    "radix2_classes": _radix(2, 13)[:3],                                      # 1024 classes, 128 a tile
    "radix4_classes": _radix(4, 7)[:2],                                       # 1024 classes, 64 a tile
    "three_slabs": [(3, 2, 2, 4096), (6, 2, 2, 2048), (12, 2, 2, 1024)],      # P = 3
    "classes_1536": [(1, 2, 2, 6144), (2, 2, 2, 3072), (4, 2, 2, 1536)],      # Q not a power of two
    "runs_of_205": [(1, 2, 2, 4100), (2, 2, 2, 2050)],                        # T = 205
    "expand_contract": [(1, 4, 2, 4096), (4, 2, 4, 1024)],                    # b != c
    "merged_slabs": _radix(2, 13)[5:],                                        # 32 slabs of 256
    "wide_slabs": [(4 ** k, 4, 4, 2 ** 13 // 4 ** k) for k in range(6)][2:],  # 16 slabs of 2048
}


@pytest.mark.parametrize("name", sorted(RUNS))
def test_tiles_reproduce_the_chain(name):
    pats = RUNS[name]
    tile = rule_tile(pats)
    assert tile is not None
    P, Q, T = tile
    wl = datagen.Workload("tiles", pats, 3, [1.0 / np.sqrt(p[2]) for p in pats], 50 + len(name))
    X, Ws = datagen.draw(wl)
    Xd, Wd = oracle.widen(X), [oracle.widen(w) for w in Ws]
    Y = run_tiled(pats, Xd, Wd, P, Q, T)
    ref = oracle.ks_chain_matmul(pats, Wd, Xd)
    assert np.max(np.abs(Y - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("name", sorted(RUNS))
def test_planner_reports_the_rule_tile(name):
    """The library plans the run as one launch on the rule's tile (slabs
    described by their count and width, class tiles by P, Q and T)."""
    pats = RUNS[name]
    P, Q, T = rule_tile(pats)
    assert libks.ks_chain_groups(pats, 3, libks.DTYPE_F32) == [list(range(len(pats)))]
    desc = libks.ks_chain_describe(pats, 3, libks.DTYPE_F32)
    if Q == 1:
        n_in = pats[0][0] * pats[0][2] * pats[0][3]
        m = re.search(r"(\d+) slabs of (\d+) values", desc)
        assert m and (int(m.group(1)), int(m.group(2))) == (P, n_in // P), desc
    else:
        m = re.search(r"(\d+) slabs x (\d+) classes, (\d+) classes a tile", desc)
        assert m and tuple(int(v) for v in m.groups()) == (P, Q, T), desc
