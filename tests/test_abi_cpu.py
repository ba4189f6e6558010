"""libks host logic without a GPU: the library loads, exports every entry
point include/ks.h declares, and rejects bad arguments with the documented
status before any HIP call (these calls never reach the device)."""
import os
import re
import subprocess

import numpy as np
import pytest

from kronecker_sparse_structured_amd import libks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ks.h")

# Fake, well-aligned device addresses far apart; validation never dereferences.
XP, WP, YP, WSP = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ks_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return libks.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"ks_matmul", "ks_chain_matmul", "ks_chain_workspace_size"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", libks.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ks_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_status_strings_and_version():
    for i, name in enumerate(libks.STATUS):
        assert libks.ks_status_string(i).startswith(name)
    assert libks.ks_status_string(999) == "KS_ERR_UNKNOWN"
    assert "gfx950" in libks.ks_version()


def st(p, W=WP, X=XP, Y=YP, batch=4, dtype=libks.DTYPE_F32, **kw):
    return libks.ks_matmul_ex(p, W, X, Y, batch, dtype, stream=0, check=False, **kw)


@pytest.mark.parametrize("p", [(0, 1, 1, 1), (1, 0, 1, 1), (1, 1, -3, 1), (1, 1, 1, 0),
                               (1 << 16, 1, 1 << 15, 1), (2, 1 << 30, 2, 1), (1, 46341, 46341, 1)])
def test_bad_pattern(p):
    assert st(p) == libks.KS_ERR_PATTERN


def test_bad_batch():
    assert st((2, 2, 2, 2), batch=-1) == libks.KS_ERR_BATCH
    assert st((2, 2, 2, 2), batch=1 << 31) == libks.KS_ERR_BATCH


def test_bad_dtype():
    assert st((2, 2, 2, 2), dtype=3) == libks.KS_ERR_DTYPE
    assert st((2, 2, 2, 2), dtype=-1) == libks.KS_ERR_DTYPE


def test_empty_batch_is_noop_even_with_null_pointers():
    assert st((2, 3, 4, 5), W=None, X=None, Y=None, batch=0) == libks.KS_OK
    assert libks.ks_matmul((2, 3, 4, 5), None, None, None, 0, libks.DTYPE_F32, stream=0, check=False) == 0


def test_null_pointers():
    for kw in ({"W": None}, {"X": None}, {"Y": None}):
        assert st((2, 2, 2, 2), **kw) == libks.KS_ERR_NULL


def test_alignment():
    assert st((2, 2, 2, 2), X=XP + 2) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), Y=YP + 1) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), W=WP + 3, dtype=libks.DTYPE_BF16) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), X=XP + 1, dtype=libks.DTYPE_BF16) == libks.KS_ERR_ALIGN
    # bf16 X on a 2-byte boundary and fp32 Y on a 4-byte boundary are fine for
    # validation; the call then proceeds to the device, which is not tested here.


def test_overlap():
    p = (2, 4, 4, 2)  # n_in = n_out = 16, batch 4 -> 256 bytes each
    assert st(p, Y=XP) == libks.KS_ERR_OVERLAP
    assert st(p, Y=XP + 252) == libks.KS_ERR_OVERLAP      # last 4 bytes of X
    assert st(p, Y=WP + 4) == libks.KS_ERR_OVERLAP
    assert st(p, Y=XP - 256 + 4) == libks.KS_ERR_OVERLAP  # Y tail reaches X head


def test_options():
    assert st((2, 2, 2, 2), kernel=99) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), rows_per_block=-1) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), reserved=[1]) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), reserved=[0, 0, 1]) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), mfma_loaders=3) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), mfma_loaders=-1) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), mfma_tile=-1) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), mfma_tile=libks.MFMA_TILES + 1) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), store_waves=3) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), store_waves=-1) == libks.KS_ERR_INVALID
    # a forced family that cannot run the pattern is refused on the host
    assert st((2, 3, 5, 2), kernel="valu") == libks.KS_ERR_UNSUPPORTED
    assert st((2, 3, 5, 2), kernel="mfma") == libks.KS_ERR_UNSUPPORTED


def cst(ps, batch=4, dtype=libks.DTYPE_F32, ws=WSP, ws_bytes=1 << 30, flags=0, Ws=None, X=XP, Y=YP, n=None):
    Ws = Ws if Ws is not None else [WP + 0x100000 * i for i in range(len(ps))]
    return libks.ks_chain_matmul(ps, Ws, X, Y, batch, dtype, ws, ws_bytes, flags, stream=0, n=n, check=False)


def test_chain_validation():
    ok = [(1, 4, 2, 4), (4, 2, 2, 2)]
    assert cst(ok, n=0) == libks.KS_ERR_CHAIN_MISMATCH
    assert cst([(1, 4, 2, 4), (4, 2, 3, 2)]) == libks.KS_ERR_CHAIN_MISMATCH
    assert cst(ok, dtype=7) == libks.KS_ERR_DTYPE
    assert cst(ok, dtype=libks.DTYPE_BF16W, X=XP + 2) == libks.KS_ERR_ALIGN     # fp32 X, bf16 weights
    assert cst(ok, flags=7) == libks.KS_ERR_INVALID
    assert cst(ok, batch=-2) == libks.KS_ERR_BATCH
    assert cst([(1, 4, 0, 4)]) == libks.KS_ERR_PATTERN
    assert cst(ok, batch=0, X=None, Y=None, ws=None, ws_bytes=0) == libks.KS_OK
    assert cst(ok, X=None) == libks.KS_ERR_NULL
    assert cst(ok, Ws=[WP, None]) == libks.KS_ERR_NULL
    need = libks.ks_chain_workspace_size(ok, 4, libks.DTYPE_F32, libks.CHAIN_NO_FUSE)
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=None, ws_bytes=need) == libks.KS_ERR_WORKSPACE
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws_bytes=need - 1) == libks.KS_ERR_WORKSPACE
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=WSP + 8, ws_bytes=need) == libks.KS_ERR_ALIGN
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=XP, ws_bytes=need) == libks.KS_ERR_OVERLAP
    assert cst(ok, Y=XP) == libks.KS_ERR_OVERLAP
    assert cst(ok, Y=WP + 0x100000) == libks.KS_ERR_OVERLAP
    assert cst(ok, X=XP + 2) == libks.KS_ERR_ALIGN


def test_chain_workspace_sizes():
    f32, nf = libks.DTYPE_F32, libks.CHAIN_NO_FUSE
    assert libks.ks_chain_workspace_size([(2, 3, 4, 5)], 10, f32, nf) == 0
    # two factors: one fp32 intermediate of batch x 16, rounded up to 256 bytes
    two = [(1, 4, 2, 4), (4, 2, 2, 2)]
    assert libks.ks_chain_workspace_size(two, 10, f32, nf) == 768
    assert libks.ks_chain_workspace_size(two, 0, f32, nf) == 0
    # three or more: two ping-pong buffers of the widest intermediate
    three = [(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)]   # 6 -> 18 -> 12 -> 8
    assert libks.ks_chain_workspace_size(three, 100, f32, nf) == 2 * 7424
    # bf16 chains keep fp32 intermediates
    assert libks.ks_chain_workspace_size(two, 10, libks.DTYPE_BF16, nf) == 768
    # fp32 X with bf16 weights: the same fp32 intermediates
    assert libks.ks_chain_workspace_size(two, 10, libks.DTYPE_BF16W, nf) == 768
    st_, _ = libks.ks_chain_workspace_size(two, 10, 5, nf, check=False)
    assert st_ == libks.KS_ERR_DTYPE


def test_plan_describe():
    # the butterfly's first factor: fp32 follows the fitted table (the VALU
    # kernel measured faster there), bf16 the general rule (matrix cores,
    # segmented tiles)
    assert libks.ks_plan_describe((1, 16, 16, 4096), 4096, libks.DTYPE_F32).startswith("valu")
    assert libks.ks_plan_describe((1, 16, 16, 4096), 4096, libks.DTYPE_BF16).startswith("mfma")
    assert "segmented" in libks.ks_plan_describe((1, 16, 16, 4096), 4096, libks.DTYPE_BF16)
    assert libks.ks_plan_describe((1, 8, 8, 4096), 4096, libks.DTYPE_F32).startswith("valu lane")
    assert libks.ks_plan_describe((4096, 8, 8, 1), 4096, libks.DTYPE_F32).startswith("valu slab")
    assert "outputs/tile=64 of 128" in libks.ks_plan_describe((1, 128, 128, 32), 4096, libks.DTYPE_F32)
    assert libks.ks_plan_describe((2, 3, 5, 7), 10, libks.DTYPE_F32).startswith("generic")


def test_chain_describe():
    """The library's own label of each launch group: whole radix-2/4
    butterflies on 1024- or 4096-wide rows name the register-resident kernel
    (with their digit order), other runs the digit-pass kernel, pairs their
    family, single factors their tile plan."""
    r4 = [(4 ** k, 4, 4, 4 ** (5 - k)) for k in range(6)]
    d = libks.ks_chain_describe(r4, 16384, libks.DTYPE_F32)
    assert d.startswith("[0..5] register-resident butterfly: 6 radix-4 factors in 6 passes (descending)")
    assert "(ascending)" in libks.ks_chain_describe(r4[::-1], 7, libks.DTYPE_BF16)
    r2 = [(2 ** k, 2, 2, 2 ** (9 - k)) for k in range(10)]
    assert "10 radix-2 factors in 5 passes" in libks.ks_chain_describe(r2, 5, libks.DTYPE_BF16W)
    # n = 256 and a chain that is not a whole butterfly keep the digit-pass kernel
    r4s = [(4 ** k, 4, 4, 4 ** (3 - k)) for k in range(4)]
    assert libks.ks_chain_describe(r4s, 100, libks.DTYPE_F32).startswith("[0..3] digit-pass chain")
    assert libks.ks_chain_describe(r4[:5], 100, libks.DTYPE_F32).startswith("[0..4] digit-pass chain")
    bf = [(1, 16, 16, 4096), (16, 16, 16, 256), (256, 16, 16, 16), (4096, 16, 16, 1)]
    parts = libks.ks_chain_describe(bf, 4096, libks.DTYPE_F32).split("; ")
    assert [p.split("]")[0] + "]" for p in parts] == ["[0..0]", "[1..1]", "[2..3]"]
    assert parts[2].startswith("[2..3] slab pair")
    assert libks.ks_chain_describe(bf, 4096, libks.DTYPE_F32, libks.CHAIN_NO_FUSE).count(";") == 3
    with pytest.raises(libks.KSError):
        libks.ks_chain_describe([(1, 4, 4, 16), (1, 4, 4, 8)], 10, libks.DTYPE_F32)


def _closure_brute(f, g):
    """Closed components of the intermediate of f then g, by search over the
    intermediate indices (independent of the library's union-find)."""
    a1, b1, c1, d1 = f
    a2, b2, c2, d2 = g
    n = a1 * b1 * d1
    assert n == a2 * c2 * d2
    comp = [-1] * n
    comps = []
    for s in range(n):
        if comp[s] >= 0:
            continue
        stack, members = [s], []
        comp[s] = len(comps)
        while stack:
            m = stack.pop()
            members.append(m)
            al1, rest = divmod(m, b1 * d1)
            de1 = rest % d1
            al2, rest2 = divmod(m, c2 * d2)
            de2 = rest2 % d2
            nbrs = [al1 * b1 * d1 + be * d1 + de1 for be in range(b1)]
            nbrs += [al2 * c2 * d2 + ga * d2 + de2 for ga in range(c2)]
            for q in nbrs:
                if comp[q] < 0:
                    comp[q] = comp[s]
                    stack.append(q)
        comps.append(members)
    big = max(comps, key=len)
    fgroups = {(m // (b1 * d1), m % d1) for m in big}
    ggroups = {(m // (c2 * d2), m % d2) for m in big}

    def shortest_run(idx):
        idx = sorted(idx)
        best, run = len(idx), 1
        for i in range(1, len(idx) + 1):
            if i < len(idx) and idx[i] == idx[i - 1] + 1:
                run += 1
            else:
                best, run = min(best, run), 1
        return best

    c0 = comps[0]
    f0 = {(m // (b1 * d1), m % d1) for m in c0}
    g0 = {(m // (c2 * d2), m % d2) for m in c0}
    xin = [al * c1 * d1 + ga * d1 + de for al, de in f0 for ga in range(c1)]
    yout = [al * b2 * d2 + be * d2 + de for al, de in g0 for be in range(b2)]
    in_run = shortest_run(xin)
    tile = min(len(comps), max(1, -(-4 // in_run)))
    weights = len(fgroups) * b1 * c1 + len(ggroups) * b2 * c2
    return {"components": len(comps), "mid": len(big), "inputs": len(fgroups) * c1,
            "outputs": len(ggroups) * b2, "weights": weights, "in_run": in_run,
            "out_run": shortest_run(yout), "tile_components": tile, "tile_weights": tile * weights,
            "uniform": int(len({len(c) for c in comps}) == 1)}


def test_pair_closure():
    """The closure rule on the chains the pages name (figures derived by hand:
    the GPT-2 MLP pair splits each 4096-value intermediate into 8 closed
    components of 512 with 32 KiB + 16 KiB of fp32 weights; each butterfly
    pair of the 65,536-point chain into 256 of 256, whose X indices sit 256
    apart; a Monarch pair is one component, the whole row)."""
    c = libks.ks_pair_closure((1, 64, 16, 64), (64, 8, 8, 8))
    assert (c["components"], c["mid"], c["weights"] * 4) == (8, 512, 48 * 1024)
    c = libks.ks_pair_closure((1, 16, 16, 4096), (16, 16, 16, 256))
    assert (c["components"], c["mid"], c["in_run"], c["tile_components"]) == (256, 256, 1, 4)
    c = libks.ks_pair_closure((256, 16, 16, 16), (4096, 16, 16, 1))
    assert (c["components"], c["in_run"], c["tile_components"], c["tile_weights"]) == (256, 256, 1, 8192)
    c = libks.ks_pair_closure((32, 32, 32, 1), (1, 32, 32, 32))
    assert (c["components"], c["mid"], c["weights"]) == (1, 1024, 65536)
    with pytest.raises(libks.KSError):
        libks.ks_pair_closure((1, 4, 4, 16), (1, 4, 4, 8))           # 64 -> 32: chain mismatch
    with pytest.raises(libks.KSError):
        libks.ks_pair_closure((1, 8192, 1, 1024), (1024, 8, 8192, 1))  # 8 M intermediates: not analysed


def test_pair_closure_brute_force():
    """Every field against an independent search on random small pairs,
    uneven sizes included."""
    rng = np.random.default_rng(7)
    checked = 0
    while checked < 60:
        a1, b1, d1 = (int(v) for v in rng.integers(1, 7, size=3))
        n = a1 * b1 * d1
        divs = [v for v in range(1, n + 1) if n % v == 0]
        c2 = int(rng.choice(divs))
        rest = n // c2
        d2 = int(rng.choice([v for v in range(1, rest + 1) if rest % v == 0]))
        a2 = rest // d2
        f = (a1, b1, int(rng.integers(1, 6)), d1)
        g = (a2, int(rng.integers(1, 6)), c2, d2)
        assert libks.ks_pair_closure(f, g) == _closure_brute(f, g), (f, g)
        checked += 1


def test_chain_plan():
    three = [(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)]
    assert libks.ks_chain_plan(three, 10, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [1, 1, 1]
    assert libks.ks_chain_groups(three, 10, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [[0], [1], [2]]
    # small blocks, rows of at most 4096: the whole chain is one row-resident launch
    assert libks.ks_chain_groups(three, 10, libks.DTYPE_F32, libks.CHAIN_AUTO) == [[0, 1, 2]]


def test_chain_plan_row_resident_runs():
    """Runs of small-block factors (b * c <= 16) whose rows fit on chip
    become one launch; a factor with larger blocks or rows over 4096
    elements ends the run."""
    radix2 = [(2 ** k, 2, 2, 2 ** (11 - k)) for k in range(12)]       # n = 4096
    assert libks.ks_chain_groups(radix2, 100, libks.DTYPE_F32) == [list(range(12))]
    assert libks.ks_chain_groups(radix2, 100, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [[k] for k in range(12)]
    wide = [(2 ** k, 2, 2, 2 ** (12 - k)) for k in range(13)]          # n = 8192: two tiled runs
    assert libks.ks_chain_groups(wide, 100, libks.DTYPE_F32) == [list(range(3)), list(range(3, 13))]
    mixed = [(64, 4, 4, 4), (1, 64, 16, 64), (256, 4, 4, 4), (256, 4, 4, 4)]
    assert libks.ks_chain_groups(mixed, 100, libks.DTYPE_F32) == [[0], [1], [2, 3]]
    big_blocks = [(1, 16, 8, 256), (16, 2, 2, 128), (32, 2, 2, 64)]    # 16 x 8 blocks first
    for dt in (libks.DTYPE_F32, libks.DTYPE_BF16):
        assert libks.ks_chain_groups(big_blocks, 100, dt) == [[0], [1, 2]]
    assert libks.ks_chain_groups([(16, 8, 8, 8), (128, 8, 8, 1)], 100, libks.DTYPE_F32) == [[0], [1]]


def test_chain_plan_tiled_runs():
    """Rows wider than 4096 elements: a run of small-block factors is cut
    into slabs (P divides every a) when one slab fits in 4096 values, as
    many consecutive slabs a tile as stay within 256 values; or else into one
    slab and groups of T of its Q index classes (Q divides every d), at most
    1024 values of a row a tile, in runs of at least 32 elements (128-byte
    lines of fp32); the run ends where no such tile exists, or earlier when
    the rest of the chain is a whole radix-2/4 butterfly on every slab of
    1024 or 4096 values (the register-resident kernel, one slab's weights a
    workgroup)."""
    f32 = libks.DTYPE_F32
    radix2 = [(2 ** k, 2, 2, 2 ** (15 - k)) for k in range(16)]      # n = 65,536
    assert libks.ks_chain_groups(radix2, 4096, f32) == [list(range(4)), list(range(4, 16))]
    desc = libks.ks_chain_describe(radix2, 4096, f32)
    assert "1 slabs x 4096 classes, 64 classes a tile" in desc, desc
    assert "register-resident butterfly on each of 16 slabs of 4096 values" in desc, desc
    # reversed: the resident run first, then the class tile
    assert libks.ks_chain_groups(radix2[::-1], 4096, f32) == [list(range(12)), list(range(12, 16))]
    # the longest resident rest: 12 factors on 4096-value slabs after two, not
    # 10 on 1024-value slabs after four
    radix2_16k = [(2 ** k, 2, 2, 2 ** (13 - k)) for k in range(14)]
    assert libks.ks_chain_groups(radix2_16k, 16384, f32) == [[0, 1], list(range(2, 14))]
    radix4 = [(4 ** k, 4, 4, 4 ** (7 - k)) for k in range(8)]         # n = 65,536
    assert libks.ks_chain_groups(radix4, 4096, f32) == [[0, 1], [2, 3, 4, 5, 6, 7]]
    three_slabs = [(3, 2, 2, 4096), (6, 2, 2, 2048), (12, 2, 2, 1024)]
    assert "3 slabs x 1024 classes, 128 classes a tile" in libks.ks_chain_describe(three_slabs, 7, f32)
    assert "1 slabs x 2050 classes, 205 classes a tile" in libks.ks_chain_describe(
        [(1, 2, 2, 4100), (2, 2, 2, 2050)], 7, f32)
    assert "5 slabs of 1024 values" in libks.ks_chain_describe(
        [(5, 2, 2, 512), (10, 2, 2, 256), (20, 2, 2, 128)], 7, f32)
    # radix-4 on n = 32,768: a third factor would leave 512 classes of 64
    # values (runs of 16 in a 1024-value tile), so the run stops at two; the
    # last four factors share 16 slabs of 2048 values
    radix4_odd = [(4 ** k, 4, 4, 2 ** 13 // 4 ** k) for k in range(6)]
    assert libks.ks_chain_groups(radix4_odd, 7, f32) == [[0, 1], [2, 3, 4, 5]]
    assert "16 slabs of 2048 values" in libks.ks_chain_describe(radix4_odd, 7, f32)


def test_chain_plan_fuses_known_pairs():
    """The planner fuses the GPT-2 pair (rows shared by groups of beta0), the
    butterfly's last two factors (the second works inside the first's output
    slabs), for fp32 rows a factor with the next one of the strided family
    (a, 16, 16, 16 e) -> (16 a, 16, 16, e), and Monarch pairs
    (M, N, N, 1) -> (1, M, M, N); nothing with NO_FUSE."""
    gpt2 = [(1, 64, 16, 64), (64, 8, 8, 8)]
    bfly = [(16 ** k, 16, 16, 16 ** (3 - k)) for k in range(4)]
    for dt in (libks.DTYPE_F32, libks.DTYPE_BF16):
        assert libks.ks_chain_groups(gpt2, 1000, dt) == [[0, 1]]
        assert libks.ks_chain_groups(bfly, 1000, dt, libks.CHAIN_NO_FUSE) == [[0], [1], [2], [3]]
    # the 65,536-point butterfly: e = 256 and 16 between its first three
    # factors, too far apart for the strided pair
    for dt in (libks.DTYPE_F32, libks.DTYPE_BF16, libks.DTYPE_BF16W):
        assert libks.ks_chain_groups(bfly, 1000, dt) == [[0], [1], [2, 3]]
    # strided family: e = 4 or 8; fp32 rows; the spare buffer for unaligned X or Y
    for e in (4, 8):
        pair = [(2, 16, 16, 16 * e), (32, 16, 16, e)]
        assert libks.ks_chain_groups(pair, 7, libks.DTYPE_F32) == [[0, 1]]
        assert libks.ks_chain_groups(pair, 7, libks.DTYPE_BF16W) == [[0, 1]]
        assert libks.ks_chain_groups(pair, 7, libks.DTYPE_BF16) == [[0], [1]]
        assert libks.ks_chain_workspace_size(pair, 7, libks.DTYPE_F32) == (7 * 512 * e * 4 + 255) // 256 * 256
    assert libks.ks_chain_groups([(2, 16, 16, 256), (32, 16, 16, 16)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(2, 16, 16, 32), (32, 16, 16, 2)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(2, 16, 16, 64), (32, 8, 16, 4)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_workspace_size(bfly, 100, libks.DTYPE_F32) == 2 * 100 * 65536 * 4
    # slab family: (a, 16, 16, 16) -> (16 a, 16, 16, 1) for any a; other shapes stay apart
    assert libks.ks_chain_groups([(3, 16, 16, 16), (48, 16, 16, 1)], 7, libks.DTYPE_F32) == [[0, 1]]
    assert libks.ks_chain_groups([(4, 16, 16, 16), (64, 16, 8, 2)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(4, 8, 16, 16), (32, 16, 16, 1)], 7, libks.DTYPE_F32) == [[0], [1]]

    # Monarch family: (M, N, N, 1) -> (1, M, M, N) with M, N in {16, 32}, every
    # dtype; the spare buffer for unaligned X or Y; other shapes stay apart
    for M in (16, 32):
        for N in (16, 32):
            pair = [(M, N, N, 1), (1, M, M, N)]
            for dt in (libks.DTYPE_F32, libks.DTYPE_BF16, libks.DTYPE_BF16W):
                assert libks.ks_chain_groups(pair, 7, dt) == [[0, 1]]
                assert libks.ks_chain_groups(pair, 7, dt, libks.CHAIN_NO_FUSE) == [[0], [1]]
            assert libks.ks_chain_workspace_size(pair, 7, libks.DTYPE_F32) == (7 * M * N * 4 + 255) // 256 * 256
    assert libks.ks_chain_groups([(64, 64, 64, 1), (1, 64, 64, 64)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(32, 32, 32, 1), (1, 32, 16, 64)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(32, 32, 32, 2), (2, 32, 32, 32)], 7, libks.DTYPE_F32) == [[0], [1]]

def test_one_hip_runtime_whatever_the_import_order():
    """Loading libks before torch must still leave a single HIP runtime in
    the process (torch bundles its own; libks has to bind to that one)."""
    import sys
    code = ("from kronecker_sparse_structured_amd import libks; libks.load(); "
            "print(len(libks._hip_runtimes()))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_backward_workspace_sizes():
    p = (4, 64, 16, 6)
    nnz = 4 * 64 * 16 * 6
    assert libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_F32) == (nnz * 4 + 255) // 256 * 256
    assert libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_BF16) == (nnz * 2 + 255) // 256 * 256
    assert libks.ks_matmul_dw_workspace_size(p, 1, libks.DTYPE_F32) == 0
    big = libks.ks_matmul_dw_workspace_size(p, 25216, libks.DTYPE_F32)
    assert big % 256 == 0 and big >= 2 * nnz * 4 and big <= 64 << 20
    assert libks.ks_matmul_dx_workspace_size((0, 1, 1, 1), 0, check=False)[0] == libks.KS_ERR_PATTERN
    assert libks.ks_matmul_dw_workspace_size(p, -1, 0, check=False)[0] == libks.KS_ERR_BATCH
    assert libks.ks_matmul_dw_workspace_size(p, 5, 7, check=False)[0] == libks.KS_ERR_DTYPE


def test_backward_argument_errors():
    p = (2, 4, 8, 2)
    need = libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_F32)
    dx = lambda **kw: libks.ks_matmul_dx(kw.get("p", p), kw.get("W", WP), kw.get("dY", XP), kw.get("dX", YP),
                                         kw.get("batch", 4), kw.get("dt", libks.DTYPE_F32), kw.get("ws", WSP),
                                         kw.get("wsb", need), stream=0, check=False)
    assert dx(p=(1, 0, 1, 1)) == libks.KS_ERR_PATTERN
    assert dx(batch=-2) == libks.KS_ERR_BATCH
    assert dx(dt=9) == libks.KS_ERR_DTYPE
    assert dx(batch=0, W=None, dY=None, dX=None, ws=None) == libks.KS_OK
    assert dx(W=None) == libks.KS_ERR_NULL
    assert dx(ws=None) == libks.KS_ERR_WORKSPACE
    assert dx(wsb=need - 1) == libks.KS_ERR_WORKSPACE
    assert dx(dX=YP + 2) == libks.KS_ERR_ALIGN
    assert dx(ws=WSP + 4) == libks.KS_ERR_ALIGN
    assert dx(dX=XP) == libks.KS_ERR_OVERLAP          # dX over dY
    assert dx(ws=WP) == libks.KS_ERR_OVERLAP          # workspace over W
    dw = lambda **kw: libks.ks_matmul_dw(kw.get("p", p), kw.get("dY", YP), kw.get("X", XP), kw.get("dW", WP),
                                         kw.get("batch", 1), kw.get("dt", libks.DTYPE_F32), kw.get("ws", None),
                                         kw.get("wsb", 0), stream=0, check=False)
    assert libks.ks_matmul_dw_workspace_size(p, 1, libks.DTYPE_F32) == 0    # one row range: no partial sums
    assert dw(p=(1, 1, 1, 0)) == libks.KS_ERR_PATTERN
    assert dw(batch=-1) == libks.KS_ERR_BATCH
    assert dw(dt=5) == libks.KS_ERR_DTYPE
    assert dw(dW=None) == libks.KS_ERR_NULL
    assert dw(X=None) == libks.KS_ERR_NULL
    assert dw(dW=WP + 1) == libks.KS_ERR_ALIGN
    assert dw(dW=XP) == libks.KS_ERR_OVERLAP
    big = (64, 8, 8, 8)
    need_w = libks.ks_matmul_dw_workspace_size(big, 4096, libks.DTYPE_F32)
    assert need_w > 0
    assert dw(p=big, batch=4096, ws=None, wsb=0) == libks.KS_ERR_WORKSPACE
    assert dw(p=big, batch=4096, ws=WSP, wsb=need_w - 1) == libks.KS_ERR_WORKSPACE


def test_dw_noalloc_argument_errors():
    """The no-allocation dK entry point validates like ks_matmul_dw (no
    workspace arguments), and every dK call's partial sums fit its scratch."""
    p = (2, 4, 8, 2)
    dw = lambda **kw: libks.ks_matmul_dw_noalloc(kw.get("p", p), kw.get("dY", YP), kw.get("X", XP),
                                                 kw.get("dW", WP), kw.get("batch", 1),
                                                 kw.get("dt", libks.DTYPE_F32), stream=0, check=False)
    assert dw(p=(1, 1, 1, 0)) == libks.KS_ERR_PATTERN
    assert dw(batch=-1) == libks.KS_ERR_BATCH
    assert dw(dt=5) == libks.KS_ERR_DTYPE
    assert dw(dW=None) == libks.KS_ERR_NULL
    assert dw(X=None) == libks.KS_ERR_NULL
    assert dw(dW=WP + 1) == libks.KS_ERR_ALIGN
    assert dw(X=XP + 2) == libks.KS_ERR_ALIGN
    assert dw(dW=XP) == libks.KS_ERR_OVERLAP
    scratch = 64 << 20   # KS_DW_SCRATCH_BYTES
    header = open(HEADER).read()
    assert re.search(r"#define KS_DW_SCRATCH_BYTES \(64u << 20\)", header)
    for q in [(4, 64, 16, 6), (64, 8, 8, 8), (1, 128, 128, 32), (3, 5, 7, 2), (4096, 16, 16, 1),
              (1, 16, 16, 4096), (2, 128, 128, 4), (1, 4, 4, 64)]:
        for batch in (1, 333, 4096, 25216, 1 << 20, (1 << 31) - 1):
            for dt in (libks.DTYPE_F32, libks.DTYPE_BF16):
                assert libks.ks_matmul_dw_workspace_size(q, batch, dt) <= scratch, (q, batch, dt)


def test_planner_follows_fitted_table():
    """For every pattern of the measured sweep, the planner picks the family
    the sweep found fastest (the table generated into ks_plan_table.inc);
    the family's name starts the plan description."""
    inc = os.path.join(ROOT, "kronecker_sparse_structured_amd", "csrc", "ks_plan_table.inc")
    prefix = {libks.KERNEL_MFMA: "mfma", libks.KERNEL_VALU: "valu", libks.KERNEL_COLUMN: "col",
              libks.KERNEL_GENERIC: "generic"}
    n = 0
    for line in open(inc):
        m = re.match(r"\{(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)(?:, (\d+))?(?:, (\d+))?\},", line)
        if not m:
            continue
        a, b, c, d, xt, wt, kernel, store = (int(v) for v in m.groups()[:8])
        tile = int(m.group(9) or 0)
        loaders = int(m.group(10) or 0)
        dt = {(0, 0): libks.DTYPE_F32, (1, 1): libks.DTYPE_BF16, (0, 1): libks.DTYPE_BF16W}[(xt, wt)]
        desc = libks.ks_plan_describe((a, b, c, d), 16384, dt)
        assert desc.startswith(prefix[kernel]), ((a, b, c, d), kernel, desc)
        if kernel == libks.KERNEL_MFMA and store:
            assert ("storers=1" in desc) == (store == libks.STORE_DEDICATED), ((a, b, c, d), store, desc)
        if kernel == libks.KERNEL_MFMA and tile:
            # candidate K: (B-register budget, b split) as listed in ks.h
            vb, split = [(32, 1), (64, 1), (128, 1), (128, 2), (64, 2), (128, 4), (64, 4)][tile - 1]
            assert "B regs=%d " % vb in desc and "outputs/tile=%d of %d " % (b // split, b) in desc, (tile, desc)
        if kernel == libks.KERNEL_MFMA:
            assert ("loaders=2" in desc) == (loaders == 2), (loaders, desc)
        n += 1
    assert n >= 51
