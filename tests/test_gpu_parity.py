"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Every case is compared on every output: the relative Frobenius error over
all of Y (the oracle streams the rows for the full-size workloads, at the
sizes and in the launch configuration the benchmark uses), plus, for single
factors, a per-element error bound (on sampled rows at full size). Every
kernel family that supports a pattern is run on the same input.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DEV, FP32_REL_TOL, chain_check, check_factor, host_values, rel_err,
                         require_gpu, run_factor, sample_rows, to_dev)
from kronecker_sparse_structured_amd import datagen, libks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    print("device:", torch.cuda.get_device_name(0), flush=True)


def try_family(p, Xt, Wt, kernel):
    """Run with a forced family; None if the family refuses the pattern."""
    a, b, c, d = p
    Y = torch.empty((Xt.shape[0], a * b * d), dtype=torch.float32, device=DEV)
    st = libks.ks_matmul_ex(p, Wt, Xt, Y, Xt.shape[0], libks.dtype_code(Xt.dtype, Wt.dtype),
                            kernel=kernel, check=False)
    if st == libks.KS_ERR_UNSUPPORTED:
        return None
    assert st == libks.KS_OK, libks.ks_status_string(st)
    return Y


ALL_FAMILIES = ["auto", "generic", "valu", "mfma", "mfma_lds", "col"]

# ---------------------------------------------------------------- small workloads


def test_tiny_factor_all_families():
    wl = datagen.get("tiny")
    X, (W,) = datagen.draw(wl)
    p = wl.patterns[0]
    Xt, Wt = to_dev(X), to_dev(W)
    ran = []
    for k in ALL_FAMILIES:
        Y = try_family(p, Xt, Wt, k)
        if Y is None:
            continue
        torch.cuda.synchronize()
        check_factor(p, X, W, Y.cpu().numpy())
        ran.append(k)
    assert "generic" in ran and "auto" in ran


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fuse", [True, False])
def test_hadamard_chain_exact(bf16, fuse):
    """Integer X in [-8, 8] through the four (2^k,2,2,2^(3-k)) factors equals
    X H16 exactly (the oracle equals X H16; pinned by scipy's Hadamard)."""
    wl = datagen.get("hadamard16")
    X, Ws = datagen.draw(wl)
    Xt = to_dev(X, bf16)
    Wts = [to_dev(W, bf16) for W in Ws]
    Y = libks.chain_matmul(Xt, Wts, wl.patterns, fuse=fuse)
    torch.cuda.synchronize()
    ref = oracle.ks_chain_matmul(wl.patterns, [host_values(W, bf16) for W in Ws], host_values(X, bf16))
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)
    import scipy.linalg
    assert np.array_equal(ref, X.astype(np.float64) @ scipy.linalg.hadamard(16))


@pytest.mark.parametrize("bf16", [False, True])
def test_integer_exact_all_families(bf16):
    """Integer data keeps every partial sum exact in fp32: all families must
    agree with the oracle bit for bit."""
    for p in [(2, 4, 4, 2), (8, 16, 16, 1), (4, 8, 8, 4), (1, 16, 16, 64), (2, 64, 16, 6),
              (4, 32, 32, 2), (1, 64, 64, 4), (2, 128, 128, 1), (16, 4, 4, 16)]:
        X, W = datagen.random_pattern_inputs(p, 37, seed=sum(p), kind="int8range")
        W = np.clip(W, -4, 4)
        Xt, Wt = to_dev(X, bf16), to_dev(W, bf16)
        ref = oracle.ks_matmul(p, host_values(W, bf16), host_values(X, bf16))
        assert np.max(np.abs(ref)) < 2 ** 24
        for k in ALL_FAMILIES:
            Y = try_family(p, Xt, Wt, k)
            if Y is None:
                continue
            torch.cuda.synchronize()
            assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref), (p, k)


# ---------------------------------------------------------------- fuzz over patterns

FUZZ = [
    (1, 1, 1, 1), (3, 2, 5, 7), (2, 3, 3, 9), (5, 4, 4, 3), (1, 16, 16, 3), (7, 8, 8, 1),
    (3, 4, 8, 2), (2, 8, 4, 4), (4, 16, 8, 8), (2, 8, 16, 12), (3, 4, 4, 40), (1, 4, 4, 200),
    (9, 16, 16, 16), (5, 8, 8, 24), (1, 32, 32, 5), (3, 64, 16, 6), (2, 16, 64, 8),
    (1, 48, 32, 4), (6, 32, 32, 1), (1, 128, 128, 2), (2, 64, 64, 3), (1, 16, 32, 130),
    (129, 4, 4, 1), (1, 4, 4, 1024), (33, 8, 8, 2),
]


@pytest.mark.parametrize("p", FUZZ, ids=lambda p: "%d_%d_%d_%d" % p)
@pytest.mark.parametrize("batch", [1, 131])
def test_fuzz_patterns_all_families(p, batch):
    X, W = datagen.random_pattern_inputs(p, batch, seed=1000 + sum(p) * batch)
    Xt, Wt = to_dev(X), to_dev(W)
    for k in ALL_FAMILIES:
        Y = try_family(p, Xt, Wt, k)
        if Y is None:
            continue
        torch.cuda.synchronize()
        check_factor(p, X, W, Y.cpu().numpy())


@pytest.mark.parametrize("p", [(2, 16, 16, 8), (64, 8, 8, 8), (256, 16, 16, 16), (2, 64, 16, 6),
                               (512, 8, 8, 1), (256, 8, 8, 2), (128, 8, 8, 4), (512, 4, 4, 2)],
                         ids=lambda p: "%d_%d_%d_%d" % p)
def test_bf16_and_mixed_inputs(p):
    X, W = datagen.random_pattern_inputs(p, 70, seed=99)
    for xb, wb in [(True, True), (False, True)]:
        Xt, Wt = to_dev(X, xb), to_dev(W, wb)
        for k in ALL_FAMILIES:
            Y = try_family(p, Xt, Wt, k)
            if Y is None:
                continue
            torch.cuda.synchronize()
            check_factor(p, X, W, Y.cpu().numpy(), bf16=xb, w_bf16=wb)


COL_PATTERNS = [(1, 16, 16, 64), (3, 16, 16, 32), (5, 16, 16, 96), (2, 32, 32, 16), (1, 32, 32, 48),
                (1, 16, 16, 4096), (16, 16, 16, 256), (1, 32, 32, 128)]


@pytest.mark.parametrize("p", COL_PATTERNS, ids=lambda p: "%d_%d_%d_%d" % p)
@pytest.mark.parametrize("batch", [1, 17, 131])
def test_column_kernel(p, batch):
    """The in-place column kernel (b = c in {16, 32}, fp32 X) on ragged row
    counts, fp32 and bf16 weights: every output against the oracle and
    within the per-element bound; equal to the tiled matrix-core kernel to
    fp32 rounding."""
    for wb in (False, True):
        X, W = datagen.random_pattern_inputs(p, batch, seed=sum(p) + batch)
        Xt, Wt = to_dev(X), to_dev(W, wb)
        Y = try_family(p, Xt, Wt, "col")
        assert Y is not None, "the column kernel refused %s" % (p,)
        torch.cuda.synchronize()
        check_factor(p, X, W, Y.cpu().numpy(), w_bf16=wb)


# ---------------------------------------------------------------- edges


def test_batch_zero_and_one():
    p = (4, 16, 16, 4)
    X, W = datagen.random_pattern_inputs(p, 1, seed=5)
    Xt, Wt = to_dev(X), to_dev(W)
    Y = run_factor(p, Xt, Wt)
    torch.cuda.synchronize()
    check_factor(p, X, W, Y.cpu().numpy())
    Y0 = torch.full((0, 256), 7.0, device=DEV)
    libks.ks_matmul(p, Wt, Xt[:0], Y0, 0, libks.DTYPE_F32)


def test_guard_bands_untouched():
    """Canaries before and after Y stay intact for every family."""
    for p, batch in [((3, 16, 16, 8), 67), ((5, 8, 8, 2), 33), ((2, 64, 16, 6), 45), ((1, 32, 32, 16), 19)]:
        a, b, c, d = p
        X, W = datagen.random_pattern_inputs(p, batch, seed=3)
        Xt, Wt = to_dev(X), to_dev(W)
        n_out = a * b * d
        for k in ALL_FAMILIES:
            guard = 4096
            buf = torch.full((guard + batch * n_out + guard,), 12345.0, device=DEV)
            Y = buf[guard:guard + batch * n_out].view(batch, n_out)
            st = libks.ks_matmul_ex(p, Wt, Xt, Y, batch, libks.DTYPE_F32, kernel=k, check=False)
            if st == libks.KS_ERR_UNSUPPORTED:
                continue
            assert st == 0
            torch.cuda.synchronize()
            h = buf.cpu().numpy()
            assert np.all(h[:guard] == 12345.0) and np.all(h[-guard:] == 12345.0), (p, k)
            check_factor(p, X, W, Y.cpu().numpy())


def test_deterministic_repeat():
    for p in [(1, 16, 16, 256), (256, 16, 16, 1), (4, 64, 16, 6), (2, 32, 32, 16)]:
        X, W = datagen.random_pattern_inputs(p, 300, seed=8)
        Xt, Wt = to_dev(X), to_dev(W)
        y1 = run_factor(p, Xt, Wt).cpu()
        y2 = run_factor(p, Xt, Wt).cpu()
        assert torch.equal(y1, y2), p


def test_non_default_stream():
    p = (16, 16, 16, 16)
    X, W = datagen.random_pattern_inputs(p, 200, seed=9)
    Xt, Wt = to_dev(X), to_dev(W)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Y = run_factor(p, Xt, Wt)
    s.synchronize()
    check_factor(p, X, W, Y.cpu().numpy())


def test_unaligned_pointers_fall_back():
    """X and Y offset by one element from 16-byte alignment still give the
    right answer (the planner picks a kernel that needs no 16-byte loads)."""
    p = (4, 16, 16, 4)
    batch = 50
    a, b, c, d = p
    X, W = datagen.random_pattern_inputs(p, batch, seed=10)
    xb = torch.empty(batch * a * c * d + 1, device=DEV)
    xb[1:] = torch.from_numpy(X.reshape(-1)).to(DEV)
    yb = torch.empty(batch * a * b * d + 1, device=DEV)
    Xt = xb[1:].view(batch, -1)
    Y = yb[1:].view(batch, -1)
    libks.ks_matmul(p, to_dev(W), Xt, Y, batch, libks.DTYPE_F32)
    torch.cuda.synchronize()
    check_factor(p, X, W, Y.cpu().numpy())


def test_nan_propagates_to_its_support():
    p = (3, 16, 16, 8)
    a, b, c, d = p
    X, W = datagen.random_pattern_inputs(p, 4, seed=11)
    al, ga, de = 1, 5, 6
    X[2, (al * c + ga) * d + de] = np.nan
    for k in ALL_FAMILIES:
        Y = try_family(p, to_dev(X), to_dev(W), k)
        if Y is None:
            continue
        bad = np.isnan(Y.cpu().numpy())
        expect = np.zeros_like(bad)
        expect[2].reshape(a, b, d)[al, :, de] = True
        assert np.array_equal(bad, expect), k


# ---------------------------------------------------------------- the named workloads


def _factor_workload(name, batch=None, rows=None, kernel="auto"):
    """One factor of a named workload. With `rows`: the relative Frobenius
    error over every output (the oracle streams the rows, nothing stored),
    and the per-element bound on those sampled rows."""
    wl = datagen.get(name)
    if batch is not None:
        wl = datagen.scaled(wl, batch)
    X, Ws = datagen.draw(wl)
    p = wl.patterns[0]
    Xt, Wt = to_dev(X), to_dev(Ws[0])
    Y = run_factor(p, Xt, Wt, kernel=kernel)
    torch.cuda.synchronize()
    if rows is None:
        return check_factor(p, X, Ws[0], Y.cpu().numpy())
    r = torch.from_numpy(rows).to(DEV)
    check_factor(p, X, Ws[0], Y.index_select(0, r).cpu().numpy(), rows=rows)
    return chain_check([p], X, Ws, Y.cpu().numpy(), False)


@pytest.mark.parametrize("batch", [1, 197, 1003])
def test_vit_mlp_small(batch):
    _factor_workload("vit_mlp", batch=batch)


def test_vit_mlp_full_size():
    """25,216 rows in the benchmark's launch configuration: every output
    within the Frobenius bound, sampled rows within the per-element bound."""
    wl = datagen.get("vit_mlp")
    _factor_workload("vit_mlp", rows=sample_rows(wl.batch))


SWEEP = datagen.square_sweep_patterns()


@pytest.mark.parametrize("p", SWEEP, ids=lambda p: "%d_%d_%d_%d" % p)
def test_square_sweep_small(p):
    _factor_workload("square_%d_%d_%d_%d" % p, batch=70)


@pytest.mark.parametrize("p", SWEEP, ids=lambda p: "%d_%d_%d_%d" % p)
def test_square_sweep_full_size(p):
    """16,384 rows: every output within the Frobenius bound, sampled rows
    within the per-element bound."""
    _factor_workload("square_%d_%d_%d_%d" % p, rows=sample_rows(16384, n=24))


def _chain_workload(name, bf16, fuse, batch=None):
    """A named chain against the oracle over every output (relative
    Frobenius error, the oracle streaming the rows)."""
    wl = datagen.get(name)
    if batch is not None:
        wl = datagen.scaled(wl, batch)
    X, Ws = datagen.draw(wl)
    Xt = to_dev(X, bf16)
    Wts = [to_dev(W, bf16) for W in Ws]
    Y = libks.chain_matmul(Xt, Wts, wl.patterns, fuse=fuse)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    del Y, Xt, Wts
    return chain_check(wl.patterns, X, Ws, Yh, bf16)


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("batch", [5, 333])
def test_gpt2_chain_small(fuse, batch):
    _chain_workload("gpt2_mlp", False, fuse, batch=batch)


@pytest.mark.parametrize("fuse", [True, False])
def test_gpt2_chain_full_size(fuse):
    """16,384 rows, fused (one launch) and one launch per factor: every output."""
    _chain_workload("gpt2_mlp", False, fuse)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("lead", [False, True])
@pytest.mark.parametrize("b0", [8, 24, 48, 64, 128])
def test_fused_pair_shapes(b0, lead, bf16):
    """The one-launch pair (1, b0, 16, 64) -> (b0, 8, 8, 8) for several b0
    (tiles of 8, 16 and 32 beta0), with a ragged row count; behind a leading
    factor in a bf16 chain the pair reads fp32 rows with bf16 weights."""
    pats = [(1, b0, 16, 64), (b0, 8, 8, 8)]
    sig = [0.25, 1.0 / np.sqrt(8.0)]
    if lead:
        pats = [(4, 16, 16, 16)] + pats
        sig = [0.25] + sig
    wl = datagen.Workload("pair", pats, 203, sig, 40 + b0)
    groups = libks.ks_chain_groups(wl.patterns, wl.batch, libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32)
    assert [len(g) for g in groups] == ([1, 2] if lead else [2])
    X, Ws = datagen.draw(wl)
    Y = libks.chain_matmul(to_dev(X, bf16), [to_dev(W, bf16) for W in Ws], wl.patterns)
    torch.cuda.synchronize()
    chain_check(wl.patterns, X, Ws, Y.cpu().numpy(), bf16)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("lead", [False, True])
@pytest.mark.parametrize("a", [1, 3, 16])
def test_slab_pair_shapes(a, lead, bf16):
    """The one-launch pair (a, 16, 16, 16) -> (16 a, 16, 16, 1) (the second
    factor works inside the first one's output slabs) for several a, with a
    ragged row count; behind a leading factor in a bf16 chain the pair reads
    fp32 rows with bf16 weights."""
    pats = [(a, 16, 16, 16), (16 * a, 16, 16, 1)]
    sig = [0.25, 0.25]
    if lead:
        pats = [(a * 16, 4, 4, 4)] + pats
        sig = [0.5] + sig
    wl = datagen.Workload("slab", pats, 203, sig, 70 + a)
    groups = libks.ks_chain_groups(wl.patterns, wl.batch, libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32)
    assert [len(g) for g in groups] == ([1, 2] if lead else [2])
    X, Ws = datagen.draw(wl)
    Y = libks.chain_matmul(to_dev(X, bf16), [to_dev(W, bf16) for W in Ws], wl.patterns)
    torch.cuda.synchronize()
    chain_check(wl.patterns, X, Ws, Y.cpu().numpy(), bf16)


@pytest.mark.parametrize("bf16w", [False, True])
@pytest.mark.parametrize("lead", [False, True])
@pytest.mark.parametrize("ae", [(1, 4), (2, 8), (3, 4), (64, 4), (5, 8)], ids=lambda v: "a%d_e%d" % v)
def test_strided_pair_shapes(ae, lead, bf16w):
    """The one-launch pair (a, 16, 16, 16 e) -> (16 a, 16, 16, e) (closed
    groups of 256 values e apart; e <= 8) on ragged row counts, with fp32 or
    bf16 weights (fp32 X); behind a leading factor the pair reads the
    workspace."""
    a, e = ae
    pats = [(a, 16, 16, 16 * e), (16 * a, 16, 16, e)]
    if lead:
        pats = [(a * 16 * e, 4, 4, 4)] + pats
    batch = 37 if a >= 64 else 203
    wl = datagen.Workload("strided", pats, batch, [1.0 / np.sqrt(p[2]) for p in pats], 60 + a + e)
    dt = libks.DTYPE_BF16W if bf16w else libks.DTYPE_F32
    groups = libks.ks_chain_groups(wl.patterns, wl.batch, dt)
    assert [len(g) for g in groups] == ([1, 2] if lead else [2]), groups
    X, Ws = datagen.draw(wl)
    Wts = [to_dev(W, bf16w) for W in Ws]
    Y = libks.chain_matmul(to_dev(X), Wts, wl.patterns)
    torch.cuda.synchronize()
    Xd = host_values(X, False)
    Wd = [host_values(W, bf16w) for W in Ws]
    se, sr, ma = oracle.ks_chain_err(wl.patterns, Wd, Xd, Y.cpu().numpy())
    assert np.sqrt(se / sr) <= FP32_REL_TOL, (np.sqrt(se / sr), ma)


MONARCH_DTYPES = {"f32": libks.DTYPE_F32, "bf16": libks.DTYPE_BF16, "bf16w": libks.DTYPE_BF16W}


@pytest.mark.parametrize("dt", sorted(MONARCH_DTYPES))
@pytest.mark.parametrize("lead", [False, True])
@pytest.mark.parametrize("mn", [(16, 16), (16, 32), (32, 16), (32, 32)], ids=lambda v: "m%d_n%d" % v)
def test_monarch_pair_shapes(mn, lead, dt):
    """The one-launch Monarch pair (M, N, N, 1) -> (1, M, M, N): whole rows
    in LDS, both products on the matrix cores. A ragged row count (203 rows,
    13 stages of 16) and one large enough that every workgroup runs several
    stages around its LDS ring (9001 rows); bf16 X with bf16 weights, and
    fp32 X with fp32 or bf16 weights; behind a leading factor the pair reads
    the workspace."""
    M, N = mn
    pats = [(M, N, N, 1), (1, M, M, N)]
    if lead:
        pats = [(M * N // 4, 4, 4, 1)] + pats
    code = MONARCH_DTYPES[dt]
    bf16 = dt == "bf16"
    w_bf16 = dt != "f32"
    for batch in (203, 9001):
        wl = datagen.Workload("monarch", pats, batch, [1.0 / np.sqrt(p[2]) for p in pats], 80 + M + N)
        groups = libks.ks_chain_groups(wl.patterns, wl.batch, code)
        assert [len(g) for g in groups] == ([1, 2] if lead else [2]), groups
        X, Ws = datagen.draw(wl)
        Y = libks.chain_matmul(to_dev(X, bf16), [to_dev(W, w_bf16) for W in Ws], wl.patterns)
        torch.cuda.synchronize()
        Xd = host_values(X, bf16)
        Wd = [host_values(W, w_bf16) for W in Ws]
        se, sr, ma = oracle.ks_chain_err(wl.patterns, Wd, Xd, Y.cpu().numpy())
        # the oracle takes the same bf16-rounded inputs, so only fp32
        # accumulation separates the two
        assert np.sqrt(se / sr) <= FP32_REL_TOL, (batch, np.sqrt(se / sr), ma)


@pytest.mark.parametrize("dt", sorted(MONARCH_DTYPES))
@pytest.mark.parametrize("mn", [(16, 32), (32, 32)], ids=lambda v: "m%d_n%d" % v)
def test_monarch_pair_weights_at_element_offsets(mn, dt):
    """The Monarch pair with both weight tensors one element past a 16-byte
    boundary (the API asks only for element alignment of weights): still one
    launch, and the same bits as with aligned weights."""
    M, N = mn
    pats = [(M, N, N, 1), (1, M, M, N)]
    code = MONARCH_DTYPES[dt]
    bf16 = dt == "bf16"
    w_bf16 = dt != "f32"
    wl = datagen.Workload("monarch", pats, 1001, [1.0 / np.sqrt(p[2]) for p in pats], 90 + M + N)
    X, Ws = datagen.draw(wl)
    Xd = to_dev(X, bf16)
    Wa = [to_dev(W, w_bf16) for W in Ws]
    Wo = [_offset_copy(w, 1) for w in Wa]
    assert all(w.data_ptr() % 16 != 0 for w in Wo)
    Ya = libks.chain_matmul(Xd, Wa, pats)
    Yo = libks.chain_matmul(Xd, Wo, pats)
    torch.cuda.synchronize()
    assert libks.ks_chain_groups(pats, wl.batch, code) == [[0, 1]]
    assert np.array_equal(Ya.cpu().numpy(), Yo.cpu().numpy())
    se, sr, ma = oracle.ks_chain_err(pats, [host_values(W, w_bf16) for W in Ws], host_values(X, bf16),
                                     Yo.cpu().numpy())
    assert np.sqrt(se / sr) <= FP32_REL_TOL, (np.sqrt(se / sr), ma)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fuse", [True, False])
def test_monarch_chain_full_size(bf16, fuse):
    """65,536 rows of 1,024 through the Monarch pair (32 blocks of 32 x 32,
    then their mixing), in one launch and one launch per factor: every
    output."""
    _chain_workload("monarch_n1024", bf16, fuse)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("store", [libks.STORE_COMPUTE, libks.STORE_DEDICATED])
@pytest.mark.parametrize("p", [(1, 128, 128, 32), (4, 128, 128, 8), (8, 128, 128, 4), (2, 64, 64, 32), (8, 64, 64, 8)],
                         ids=lambda v: "%d_%d_%d_%d" % v)
def test_mfma_two_loader_waves(p, store, bf16):
    """The matrix-core kernel with two loader waves (each issuing every other
    LDS-DMA instruction of a stage) on segmented and contiguous tiles, with
    either store schedule and a ragged row count: the same result as one
    loader wave, and the oracle's. Blocks narrower than 64 refuse it."""
    a, b, c, d = p
    batch = 1001
    X, W = datagen.random_pattern_inputs(p, batch, 120 + a)
    Xt, Wt = to_dev(X, bf16), to_dev(W, bf16)
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    outs = []
    for loaders in (1, 2):
        Y = torch.full((batch, a * b * d), float("nan"), device=DEV)
        st = libks.ks_matmul_ex(p, Wt, Xt, Y, batch, dt, kernel="mfma", store_waves=store, mfma_loaders=loaders,
                                check=False)
        if st == libks.KS_ERR_UNSUPPORTED and store == libks.STORE_DEDICATED:
            pytest.skip("this tile has no room for a storer wave")
        assert st == 0, st
        torch.cuda.synchronize()
        outs.append(Y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    check_factor(p, X, W, outs[1], bf16=bf16)
    Y = torch.empty((10, 4 * 64 * 6), device=DEV)
    Xs, Ws = datagen.random_pattern_inputs((4, 64, 16, 6), 10, 3)
    assert libks.ks_matmul_ex((4, 64, 16, 6), to_dev(Ws), to_dev(Xs), Y, 10, libks.DTYPE_F32, kernel="mfma",
                              mfma_loaders=2, check=False) == libks.KS_ERR_UNSUPPORTED


def _radix(r, L):
    """Factors (r^k, r, r, r^(L-1-k)), k = 0..L-1: a radix-r butterfly on n = r^L."""
    return [(r ** k, r, r, r ** (L - 1 - k)) for k in range(L)]


# chains the planner runs as one row-resident launch: (patterns, rows)
ROW_CHAINS = {
    "radix2_n1024": (_radix(2, 10), 1000),
    "radix2_n4096": (_radix(2, 12), 5),
    "radix4_n4096": (_radix(4, 6), 37),
    "radix4_n64": (_radix(4, 3), 1000),
    "uneven_blocks": ([(4, 2, 8, 16), (8, 8, 2, 8), (32, 1, 16, 1)], 77),
    "odd_c3": ([(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)], 203),
    # square power-of-two blocks (several factors per LDS round trip): the
    # reversed butterfly, mixed radix, a digit mixed twice in a row, digits
    # out of order, the 16-point Hadamard shape at a ragged row count
    "radix2_reversed_n1024": (_radix(2, 10)[::-1], 333),
    "radix4_reversed_n256": (_radix(4, 4)[::-1], 1001),
    "mixed_radix_n64": ([(1, 4, 4, 16), (4, 2, 2, 8), (8, 2, 2, 4), (16, 2, 2, 2), (32, 2, 2, 1)], 257),
    "repeated_digit_n32": ([(4, 2, 2, 4), (4, 2, 2, 4), (2, 2, 2, 8), (8, 4, 4, 1), (16, 2, 2, 1)], 1025),
    "digits_out_of_order_n64": ([(4, 2, 2, 8), (4, 4, 4, 4), (32, 2, 2, 1), (1, 4, 4, 16), (2, 2, 2, 16),
                                 (8, 2, 2, 4)], 515),
    "radix2_n16": (_radix(2, 4), 3001),
    # square blocks off the power-of-two path: the general kernel, in place
    "square_in_place_n72": ([(3, 2, 2, 12), (6, 2, 2, 6), (12, 2, 2, 3)], 333),
}


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("name", sorted(ROW_CHAINS))
def test_row_chain(name, bf16):
    """A whole chain of small blocks in one launch, rows resident in LDS
    (widths up to 4096, ragged row counts, c = 3 on the general path, square
    power-of-two blocks on the several-factors-per-pass path); the same
    chain one launch per factor agrees with it and with the oracle."""
    pats, batch = ROW_CHAINS[name]
    wl = datagen.Workload("rowchain", pats, batch, [1.0 / np.sqrt(p[2]) for p in pats], 90 + len(pats))
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    assert libks.ks_chain_groups(pats, batch, dt) == [list(range(len(pats)))]
    X, Ws = datagen.draw(wl)
    Xt, Wts = to_dev(X, bf16), [to_dev(W, bf16) for W in Ws]
    Y = libks.chain_matmul(Xt, Wts, pats)
    Yu = libks.chain_matmul(Xt, Wts, pats, fuse=False)
    torch.cuda.synchronize()
    chain_check(pats, X, Ws, Y.cpu().numpy(), bf16)
    chain_check(pats, X, Ws, Yu.cpu().numpy(), bf16)


# Whole butterflies that run on the register-resident kernel: (radix, digits,
# rows); the row counts leave a ragged last block and give every workgroup
# several blocks (the DMA of block i + 1 overlaps block i).
RESIDENT = {
    "radix4_n4096": (4, 6, 4093),
    "radix2_n4096": (2, 12, 4093),
    "radix4_n1024": (4, 5, 16381),
    "radix2_n1024": (2, 10, 16381),
}


@pytest.mark.parametrize("dt", ["f32", "bf16", "bf16w"])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("name", sorted(RESIDENT))
def test_resident_butterfly(name, reverse, dt):
    """Radix-2 and radix-4 butterflies in both digit orders on the persistent
    kernel that keeps every weight in registers: all of Y against the oracle,
    fp32, bf16 and fp32 X with bf16 weights."""
    r, L, batch = RESIDENT[name]
    pats = _radix(r, L)[::-1] if reverse else _radix(r, L)
    wl = datagen.Workload("resident", pats, batch, [1.0 / np.sqrt(r)] * len(pats), 300 + 3 * L + r)
    X, Ws = datagen.draw(wl)
    bx, bw = dt == "bf16", dt != "f32"
    Xt, Wts = to_dev(X, bx), [to_dev(W, bw) for W in Ws]
    assert libks.ks_chain_groups(pats, batch, libks.dtype_code(Xt.dtype, Wts[0].dtype)) == [list(range(len(pats)))]
    Y = libks.chain_matmul(Xt, Wts, pats)
    torch.cuda.synchronize()
    se, sr, ma = oracle.ks_chain_err(pats, [host_values(W, bw) for W in Ws], host_values(X, bx), Y.cpu().numpy())
    assert np.sqrt(se / sr) <= FP32_REL_TOL, "relative Frobenius error %g (max abs %g)" % (np.sqrt(se / sr), ma)


@pytest.mark.parametrize("batch", [1, 3, 255, 16384])
def test_resident_butterfly_batches(batch):
    """The radix-4 4096-point butterfly at row counts below one block, below
    one block per workgroup, and at full size (16,384 rows), fp32; plus the
    Hadamard version bit-exact on integer rows."""
    pats = _radix(4, 6)
    wl = datagen.Workload("resident", pats, batch, [0.5] * len(pats), 400 + batch % 97)
    X, Ws = datagen.draw(wl)
    Y = libks.chain_matmul(to_dev(X), [to_dev(W) for W in Ws], pats)
    torch.cuda.synchronize()
    chain_check(pats, X, Ws, Y.cpu().numpy(), False)


@pytest.mark.parametrize("bf16", [False, True])
def test_resident_hadamard_exact(bf16):
    """The 4096-point Hadamard transform as twelve radix-2 factors of
    [[1, 1], [1, -1]] blocks on small integers: exact in fp32, so the kernel
    must match the oracle bit for bit."""
    pats = datagen.hadamard_patterns(12)
    wl = datagen.Workload("hadamard4096", pats, 77, [1.0] * len(pats), 12, x_kind="int8range", w_kind="hadamard")
    X, Ws = datagen.draw(wl)
    Y = libks.chain_matmul(to_dev(X, bf16), [to_dev(W, bf16) for W in Ws], pats).cpu().numpy()
    ref = oracle.ks_chain_matmul(pats, [host_values(W, bf16) for W in Ws], host_values(X, bf16))
    assert np.array_equal(Y.astype(np.float64), ref)


@pytest.mark.parametrize("bf16", [False, True])
def test_row_chain_unaligned_rows(bf16):
    """X and Y at 4-byte (not 16-byte) offsets: the element-wise load and
    store paths of the row-resident chain."""
    pats, batch = _radix(2, 8), 99
    wl = datagen.Workload("rowchain", pats, batch, [1.0 / np.sqrt(2.0)] * len(pats), 17)
    X, Ws = datagen.draw(wl)
    Xd = to_dev(X, bf16)
    xbuf = torch.empty(Xd.numel() + 8, dtype=Xd.dtype, device=Xd.device)
    Xo = xbuf[1:1 + Xd.numel()].view(Xd.shape)
    Xo.copy_(Xd)
    ybuf = torch.empty(batch * 256 + 8, dtype=torch.float32, device=Xd.device)
    Yo = ybuf[1:1 + batch * 256].view(batch, 256)
    libks.chain_matmul(Xo, [to_dev(W, bf16) for W in Ws], pats, out=Yo)
    torch.cuda.synchronize()
    chain_check(pats, X, Ws, Yo.cpu().numpy(), bf16)


# Runs of small-block factors whose rows are wider than 4096 elements: one
# launch per run of factors that share slabs (a divisor of every a) and
# classes of indices (a divisor of every d), a workgroup holding one slab and
# a group of classes. (patterns, rows, expected launch groups)
TILED_CHAINS = {
    # 65,536-point radix-2: 4096 classes in groups of 64, then a whole
    # 4096-point butterfly on each of 16 slabs (register-resident kernel)
    "radix2_n65536": (_radix(2, 16), 37, [list(range(4)), list(range(4, 16))]),
    # reversed: the resident slabs first (bf16 X staged), then the classes
    "radix2_n65536_reversed": (_radix(2, 16)[::-1], 37, [list(range(12)), list(range(12, 16))]),
    # 16,384-point radix-2: 4096 classes in groups of 256, then a whole
    # 4096-point butterfly on each of 4 slabs
    "radix2_n16384": (_radix(2, 14), 29, [[0, 1], list(range(2, 14))]),
    # 16,384-point radix-4: 1024 classes in groups of 64, then a whole
    # radix-4 butterfly on each of 16 slabs of 1024
    "radix4_n16384": (_radix(4, 7), 21, [[0, 1], [2, 3, 4, 5, 6]]),
    # three slabs (P = 3), each of 1024 classes taken 128 at a time
    "slabs3_classes1024": ([(3, 2, 2, 4096), (6, 2, 2, 2048), (12, 2, 2, 1024)], 19, [[0, 1, 2]]),
    # 1536 classes (not a power of two), 128 a tile
    "classes1536": ([(1, 2, 2, 6144), (2, 2, 2, 3072), (4, 2, 2, 1536)], 23, [[0, 1, 2]]),
    # 2050 classes, 205 a tile: runs that are not whole 4-element vectors
    "classes2050_runs410": ([(1, 2, 2, 4100), (2, 2, 2, 2050)], 17, [[0, 1]]),
    # five slabs of 1024 (a tile each: 5120 values do not fit)
    "slabs5_whole": ([(5, 2, 2, 512), (10, 2, 2, 256), (20, 2, 2, 128)], 33, [[0, 1, 2]]),
    # b != c: 8192 -> 16384 -> 8192 through 4 x 2 and 2 x 4 blocks
    "expand_contract": ([(1, 4, 2, 4096), (4, 2, 4, 1024)], 29, [[0, 1]]),
}


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("name", sorted(TILED_CHAINS))
def test_tiled_row_chain(name, bf16):
    """Chains on rows too wide for LDS, cut by their closure into slabs and
    groups of index classes: the planned launch groups, all of Y against the
    oracle, and the same chain one launch per factor."""
    pats, batch, groups = TILED_CHAINS[name]
    wl = datagen.Workload("tiled", pats, batch, [1.0 / np.sqrt(p[2]) for p in pats], 70 + len(pats) + batch)
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    assert libks.ks_chain_groups(pats, batch, dt) == groups
    X, Ws = datagen.draw(wl)
    Xt, Wts = to_dev(X, bf16), [to_dev(W, bf16) for W in Ws]
    Y = libks.chain_matmul(Xt, Wts, pats)
    Yu = libks.chain_matmul(Xt, Wts, pats, fuse=False)
    torch.cuda.synchronize()
    chain_check(pats, X, Ws, Y.cpu().numpy(), bf16)
    chain_check(pats, X, Ws, Yu.cpu().numpy(), bf16)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("name", ["radix2_n65536", "radix4_n65536", "radix2_n16384"])
def test_tiled_chain_full_size(name, bf16):
    """The wide butterflies at the size the benchmark times (4,096 rows of
    65,536, 16,384 rows of 16,384), in its launch configuration (two tiled
    launches whose last row blocks are ragged): every output."""
    wl = datagen.get(name)
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    assert len(libks.ks_chain_groups(wl.patterns, wl.batch, dt)) == 2
    _chain_workload(name, bf16, True)


@pytest.mark.parametrize("bf16", [False, True])
def test_tiled_row_chain_unaligned(bf16):
    """A tiled run with X and Y one element past a 16-byte boundary: the
    element-wise load and store paths of the tiles."""
    pats, batch = _radix(2, 13), 9
    wl = datagen.Workload("tiled", pats, batch, [1.0 / np.sqrt(2.0)] * len(pats), 19)
    X, Ws = datagen.draw(wl)
    Xo = _offset_copy(to_dev(X, bf16), 1)
    Yo = _offset_out(batch, 8192, 1)
    libks.chain_matmul(Xo, [to_dev(W, bf16) for W in Ws], pats, out=Yo)
    torch.cuda.synchronize()
    chain_check(pats, X, Ws, Yo.cpu().numpy(), bf16)


def test_tiled_hadamard_exact():
    """The 16,384-point Walsh-Hadamard transform (fourteen radix-2 factors of
    [[1, 1], [1, -1]] blocks) on small integers runs as two tiled launches
    and is exact in fp32: bit for bit the oracle."""
    pats = datagen.hadamard_patterns(14)
    assert libks.ks_chain_groups(pats, 11, libks.DTYPE_F32) == [[0, 1], list(range(2, 14))]
    wl = datagen.Workload("hadamard16384", pats, 11, [1.0] * len(pats), 14, x_kind="int8range", w_kind="hadamard")
    X, Ws = datagen.draw(wl)
    Y = libks.chain_matmul(to_dev(X), [to_dev(W) for W in Ws], pats).cpu().numpy()
    ref = oracle.ks_chain_matmul(pats, [host_values(W, False) for W in Ws], host_values(X, False))
    assert np.array_equal(Y.astype(np.float64), ref)


def _offset_copy(t: torch.Tensor, elems: int) -> torch.Tensor:
    """A copy of t whose storage starts `elems` elements past a 16-byte
    boundary (torch allocations are 256-byte aligned)."""
    buf = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = buf[elems:elems + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def _offset_out(rows: int, cols: int, elems: int) -> torch.Tensor:
    buf = torch.full((rows * cols + 16,), float("nan"), dtype=torch.float32, device=DEV)
    return buf[elems:elems + rows * cols].view(rows, cols)


# chains whose first group is a fused pair: (patterns, rows, seed)
FUSED_CHAINS = {
    "gpt2_pair": ([(1, 64, 16, 64), (64, 8, 8, 8)], 203, 41),
    "slab_pair_a1": ([(1, 16, 16, 16), (16, 16, 16, 1)], 77, 42),
    "slab_pair_a3": ([(3, 16, 16, 16), (48, 16, 16, 1)], 45, 43),
    "butterfly65536": (datagen.get("butterfly65536").patterns, 5, 44),
    "strided_pair_a2_e8": ([(2, 16, 16, 128), (32, 16, 16, 8)], 45, 45),
    "monarch_m32_n16": ([(32, 16, 16, 1), (1, 32, 32, 16)], 45, 46),
}


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("name", sorted(FUSED_CHAINS))
def test_fused_chain_unaligned_pointers(name, bf16):
    """The fused pair kernels with X and Y aligned only to their element
    size: X at every element offset from a 16-byte boundary that a 4-byte
    (fp32) or 2-byte (bf16) alignment allows, Y at 4 and 8 bytes past one.
    The plan keeps its fused groups and every offset matches the oracle. For
    most pairs 16-byte alignment only selects vector loads, so every offset
    gives the same bits; the strided and Monarch pairs run their two factors
    one at a time when X or Y is not 16-byte aligned, so the same bits hold
    within each of the two cases."""
    pats, batch, seed = FUSED_CHAINS[name]
    if bf16 and name.startswith("strided"):
        pytest.skip("the strided pair reads fp32 X; a bf16 chain runs these factors one at a time")
    wl = datagen.Workload("unaligned", pats, batch, [1.0 / np.sqrt(p[2]) for p in pats], seed)
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    groups = libks.ks_chain_groups(pats, batch, dt)
    assert any(len(g) == 2 for g in groups), groups
    X, Ws = datagen.draw(wl)
    Xd = to_dev(X, bf16)
    Wts = [to_dev(W, bf16) for W in Ws]
    n_out = datagen.n_out(pats[-1])
    refs = {}
    per16 = 8 if bf16 else 4
    split_when_unaligned = name.startswith("strided") or name.startswith("monarch")
    for xo in range(per16):
        for yo in ([1, 2] if xo % 2 else [0, 3]):
            Xo = _offset_copy(Xd, xo)
            Yo = _offset_out(batch, n_out, yo)
            libks.chain_matmul(Xo, Wts, pats, out=Yo)
            torch.cuda.synchronize()
            Yh = Yo.cpu().numpy()
            chain_check(pats, X, Ws, Yh, bf16)
            key = (xo == 0 and yo == 0) if split_when_unaligned else None
            if key not in refs:
                refs[key] = Yh
            else:
                # the same kernels and summation order at every such offset
                assert np.array_equal(Yh, refs[key]), (xo, yo)


def test_dw_unaligned_pointers():
    """dK for a pattern the matrix-core kernel takes, with X and dY 4 bytes
    past a 16-byte boundary: the generic kernel runs over the same row
    ranges (same workspace) and matches the oracle."""
    p = (4, 64, 16, 6)
    a, b, c, d = p
    batch = 3001
    rng = np.random.default_rng(71)
    X = rng.standard_normal((batch, a * c * d), dtype=np.float32)
    dY = rng.standard_normal((batch, a * b * d), dtype=np.float32)
    ref = oracle.ks_matmul_dw(p, host_values(dY, False), host_values(X, False))
    for xo, go in [(1, 0), (0, 3), (2, 1)]:
        dW = libks.matmul_dw(_offset_copy(to_dev(dY), go), _offset_copy(to_dev(X), xo), p)
        torch.cuda.synchronize()
        assert _rel(dW.cpu().numpy(), ref) <= FP32_REL_TOL, (xo, go)


def test_hadamard_chain_is_one_launch():
    wl = datagen.get("hadamard16")
    assert libks.ks_chain_groups(wl.patterns, wl.batch, libks.DTYPE_F32) == [[0, 1, 2, 3]]


def test_gpt2_factors_single():
    wl = datagen.get("gpt2_mlp")
    wl = datagen.scaled(wl, 257)
    X, Ws = datagen.draw(wl)
    Z = oracle.ks_matmul(wl.patterns[0], host_values(Ws[0], False), host_values(X, False)).astype(np.float32)
    for p, W, inp in [(wl.patterns[0], Ws[0], X), (wl.patterns[1], Ws[1], Z)]:
        Y = run_factor(p, to_dev(inp), to_dev(W))
        torch.cuda.synchronize()
        check_factor(p, inp, W, Y.cpu().numpy())


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fuse", [True, False])
def test_butterfly_chain_small(bf16, fuse):
    _chain_workload("butterfly65536", bf16, fuse, batch=9)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fuse", [True, False])
def test_butterfly_chain_full_size(bf16, fuse):
    """4,096 rows of 65,536, in the benchmark's launch configuration (fused)
    and one launch per factor: every output."""
    _chain_workload("butterfly65536", bf16, fuse)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_butterfly_single_factor(bf16, k):
    """Each factor alone, as the chain runs it: bf16 X for k = 0, fp32 X with
    bf16 weights after that."""
    wl = datagen.scaled(datagen.get("butterfly65536"), 40)
    X, Ws = datagen.draw(wl)
    p = wl.patterns[k]
    xb = bf16 and k == 0
    Y = run_factor(p, to_dev(X, xb), to_dev(Ws[k], bf16))
    torch.cuda.synchronize()
    check_factor(p, X, Ws[k], Y.cpu().numpy(), bf16=xb, w_bf16=bf16)


def _hip_runtime():
    """The HIP runtime library mapped into this process (None if not exactly one)."""
    import ctypes
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            name = line.split()[-1] if len(line.split()) >= 6 else ""
            if "libamdhip64.so" in name:
                paths.add(name)
    if len(paths) != 1:
        return None
    return ctypes.CDLL(paths.pop())


def test_launch_status_ignores_earlier_unrelated_error():
    """A failed HIP call made before ks_matmul (here a device attribute query
    on a device that does not exist) must not be reported as this launch's
    failure."""
    import ctypes
    wl = datagen.get("tiny")
    X, (W,) = datagen.draw(wl)
    p = wl.patterns[0]
    Xt, Wt = to_dev(X), to_dev(W)
    torch.cuda.synchronize()
    hip = _hip_runtime()
    if hip is None:
        pytest.skip("could not identify the HIP runtime of this process")
    v = ctypes.c_int(0)
    assert hip.hipDeviceGetAttribute(ctypes.byref(v), 0, 1 << 20) != 0
    for kernel in ALL_FAMILIES:
        Y = try_family(p, Xt, Wt, kernel)
        if Y is None:
            continue
        torch.cuda.synchronize()
        check_factor(p, X, W, Y.cpu().numpy())
    hip.hipGetLastError()


STORE_PATTERNS = [(4, 64, 16, 6), (1, 64, 16, 64), (16, 64, 64, 4), (128, 32, 32, 1), (1, 32, 32, 128),
                  (32, 128, 128, 1), (3, 32, 16, 5), (5, 128, 16, 2), (2, 16, 64, 2), (1, 128, 32, 4),
                  (4, 16, 16, 16), (1, 16, 32, 256)]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("p", STORE_PATTERNS, ids=lambda p: "%d_%d_%d_%d" % p)
def test_mfma_store_modes(p, bf16):
    """The MFMA kernel with Y stored by the compute waves and by a dedicated
    storer wave (double-buffered Y tile): both match the oracle on every
    output, and agree bit for bit (same MFMA sequence, only the store
    schedule differs). 48 rows per workgroup give several row steps per
    workgroup and a ragged last workgroup."""
    batch = 131
    X, W = datagen.random_pattern_inputs(p, batch, seed=sum(p) + 17)
    Xt, Wt = to_dev(X, bf16), to_dev(W, bf16)
    a, b, c, d = p
    outs = {}
    for mode in ("compute", "dedicated"):
        Y = torch.full((batch, a * b * d), float("nan"), dtype=torch.float32, device=DEV)
        st = libks.ks_matmul_ex(p, Wt, Xt, Y, batch, libks.dtype_code(Xt.dtype, Wt.dtype), kernel="mfma",
                                rows_per_block=48, store_waves=mode, check=False)
        if st == libks.KS_ERR_UNSUPPORTED:
            continue
        assert st == libks.KS_OK, libks.ks_status_string(st)
        torch.cuda.synchronize()
        outs[mode] = Y.cpu().numpy()
        check_factor(p, X, W, outs[mode], bf16=bf16)
    assert outs, "neither store mode ran"
    if len(outs) == 2:
        assert np.array_equal(outs["compute"], outs["dedicated"])


# ---------------------------------------------------------------- gradients

# (1, 128, 128, 32): dK X segments of 16 bytes, the two-loader-wave stage
BACKWARD_PATTERNS = [(2, 16, 16, 8), (4, 64, 16, 6), (64, 8, 8, 8), (3, 5, 7, 2), (2, 128, 128, 4),
                     (1, 4, 4, 64), (5, 1, 3, 2), (1, 128, 128, 32)]


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, dtype=np.float64) - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("p", BACKWARD_PATTERNS, ids=lambda p: "%d_%d_%d_%d" % p)
@pytest.mark.parametrize("dt", ["f32", "bf16", "bf16w"])
def test_backward_dx_dw(p, dt):
    """dX = dY W and dK against the fp64 oracle on a ragged batch: fp32
    everything; bf16 X and W (dY bf16 for dX); fp32 inputs with bf16 W."""
    a, b, c, d = p
    batch = 333
    rng = np.random.default_rng(500 + a * 7 + b)
    X = rng.standard_normal((batch, a * c * d), dtype=np.float32)
    W = rng.standard_normal((a, d, b, c), dtype=np.float32) / np.float32(np.sqrt(c))
    dY = rng.standard_normal((batch, a * b * d), dtype=np.float32)
    xb = dt == "bf16"
    wb = dt in ("bf16", "bf16w")
    dXg = libks.matmul_dx(to_dev(dY, xb), to_dev(W, wb), p)
    dWg = libks.matmul_dw(to_dev(dY, False), to_dev(X, xb), p)
    torch.cuda.synchronize()
    ref_dx = oracle.ks_matmul_dx(p, host_values(W, wb), host_values(dY, xb))
    ref_dw = oracle.ks_matmul_dw(p, host_values(dY, False), host_values(X, xb))
    assert _rel(dXg.cpu().numpy(), ref_dx) <= FP32_REL_TOL, "dX"
    assert _rel(dWg.cpu().numpy(), ref_dw) <= FP32_REL_TOL, "dW"


def test_backward_edges():
    """batch 0 gives dK = 0; batch 1 (no partial sums); repeated calls give
    identical bits (partial sums added in a fixed order)."""
    p = (4, 64, 16, 6)
    a, b, c, d = p
    W = torch.randn((a, d, b, c), device=DEV)
    dW = libks.matmul_dw(torch.empty((0, a * b * d), device=DEV), torch.empty((0, a * c * d), device=DEV), p)
    torch.cuda.synchronize()
    assert not dW.any()
    rng = np.random.default_rng(7)
    X = rng.standard_normal((1, a * c * d), dtype=np.float32)
    dY = rng.standard_normal((1, a * b * d), dtype=np.float32)
    dW1 = libks.matmul_dw(to_dev(dY), to_dev(X), p).cpu().numpy()
    assert _rel(dW1, oracle.ks_matmul_dw(p, host_values(dY, False), host_values(X, False))) <= FP32_REL_TOL
    X = to_dev(rng.standard_normal((3001, a * c * d), dtype=np.float32))
    dY = to_dev(rng.standard_normal((3001, a * b * d), dtype=np.float32))
    r1 = libks.matmul_dw(dY, X, p).cpu()
    r2 = libks.matmul_dw(dY, X, p).cpu()
    assert torch.equal(r1, r2)
    dx0 = libks.matmul_dx(torch.empty((0, a * b * d), device=DEV), W, p)
    assert dx0.shape == (0, a * c * d)


def test_backward_vit_full_size():
    """The ViT factor's gradients at 25,216 rows: dX and dK in full."""
    wl = datagen.get("vit_mlp")
    p = wl.patterns[0]
    X, Ws = datagen.draw(wl)
    rng = np.random.default_rng(8)
    dY = rng.standard_normal((wl.batch, wl.n_out), dtype=np.float32)
    dXg = libks.matmul_dx(to_dev(dY), to_dev(Ws[0]), p)
    dWg = libks.matmul_dw(to_dev(dY), to_dev(X), p)
    torch.cuda.synchronize()
    ref_dx = oracle.ks_matmul_dx(p, host_values(Ws[0], False), host_values(dY, False))
    assert _rel(dXg.cpu().numpy(), ref_dx) <= FP32_REL_TOL
    ref_dw = oracle.ks_matmul_dw(p, host_values(dY, False), host_values(X, False))
    assert _rel(dWg.cpu().numpy(), ref_dw) <= FP32_REL_TOL


@pytest.mark.parametrize("bf16", [False, True])
def test_kslinear_layer_gradients(bf16):
    """The autograd layer over a 2-factor chain: output and the gradients of
    L = <G, y> with respect to x and both weights, against the fp64 chain
    rule built from the oracle's single-factor functions."""
    from kronecker_sparse_structured_amd import layer
    pats = [(4, 16, 16, 8), (64, 8, 8, 1)]
    dtype = torch.bfloat16 if bf16 else torch.float32
    L = layer.KSLinear(pats, dtype=dtype, device=DEV, seed=3)
    rng = np.random.default_rng(9)
    x_np = rng.standard_normal((5, 37, L.n_in), dtype=np.float32)
    G_np = rng.standard_normal((5, 37, L.n_out), dtype=np.float32)
    x = to_dev(x_np.reshape(-1, L.n_in), bf16).reshape(5, 37, L.n_in).requires_grad_(True)
    y = L(x)
    (y * torch.from_numpy(G_np).to(DEV)).sum().backward()
    torch.cuda.synchronize()
    xs = host_values(x_np.reshape(-1, L.n_in), bf16)
    Ks = [oracle.widen(w.detach().view(torch.int16).cpu().numpy().view(np.uint16), "bf16") if bf16 else
          oracle.widen(w.detach().cpu().numpy(), "f32") for w in L.weights]
    z = oracle.ks_matmul(pats[0], Ks[0], xs)
    y_ref = oracle.ks_matmul(pats[1], Ks[1], z)
    assert _rel(y.detach().reshape(-1, L.n_out).cpu().numpy(), y_ref) <= FP32_REL_TOL
    g = G_np.reshape(-1, L.n_out).astype(np.float64)
    dK1 = oracle.ks_matmul_dw(pats[1], g, z)
    dz = oracle.ks_matmul_dx(pats[1], Ks[1], g)
    dK0 = oracle.ks_matmul_dw(pats[0], dz, xs)
    dx = oracle.ks_matmul_dx(pats[0], Ks[0], dz)
    tol = 1e-2 if bf16 else FP32_REL_TOL     # bf16 layer: gradients are rounded to bf16 on return
    assert _rel(L.weights[1].grad.float().cpu().numpy(), dK1) <= tol
    assert _rel(L.weights[0].grad.float().cpu().numpy(), dK0) <= tol
    assert _rel(x.grad.float().reshape(-1, L.n_in).cpu().numpy(), dx) <= tol



@pytest.mark.parametrize("bf16", [False, True])
def test_kslinear_inference_row_chain(bf16):
    """Without gradients the layer runs its chain through chain_matmul: a
    radix-4 butterfly on n = 256 becomes one row-resident launch, and its
    output matches the oracle chain on the layer's own weights."""
    from kronecker_sparse_structured_amd import layer
    pats = _radix(4, 4)
    assert libks.ks_chain_groups(pats, 64, libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32) == [[0, 1, 2, 3]]
    dtype = torch.bfloat16 if bf16 else torch.float32
    L = layer.KSLinear(pats, dtype=dtype, device=DEV, seed=5)
    x_np = np.random.default_rng(12).standard_normal((3, 21, L.n_in), dtype=np.float32)
    x = to_dev(x_np.reshape(-1, L.n_in), bf16).reshape(3, 21, L.n_in)
    with torch.no_grad():
        y = L(x)
    torch.cuda.synchronize()
    assert y.shape == (3, 21, L.n_out) and y.dtype == torch.float32
    Ks = [oracle.widen(w.detach().view(torch.int16).cpu().numpy().view(np.uint16), "bf16") if bf16 else
          oracle.widen(w.detach().cpu().numpy(), "f32") for w in L.weights]
    ref = oracle.ks_chain_matmul(pats, Ks, host_values(x_np.reshape(-1, L.n_in), bf16))
    assert _rel(y.reshape(-1, L.n_out).cpu().numpy(), ref) <= FP32_REL_TOL


def test_kslinear_inference_tiled_chain():
    """The layer's inference path on rows wider than LDS holds: a radix-2
    butterfly on n = 8192 runs as two tiled launches (X a view that starts
    one row into its storage), against the oracle chain on the layer's
    weights."""
    from kronecker_sparse_structured_amd import layer
    pats = _radix(2, 13)
    assert libks.ks_chain_groups(pats, 21, libks.DTYPE_F32) == [list(range(3)), list(range(3, 13))]
    L = layer.KSLinear(pats, device=DEV, seed=6)
    x_np = np.random.default_rng(13).standard_normal((22, L.n_in), dtype=np.float32)
    x = to_dev(x_np)[1:]
    with torch.no_grad():
        y = L(x)
    torch.cuda.synchronize()
    Ks = [oracle.widen(w.detach().cpu().numpy(), "f32") for w in L.weights]
    ref = oracle.ks_chain_matmul(pats, Ks, host_values(x_np[1:], False))
    assert _rel(y.cpu().numpy(), ref) <= FP32_REL_TOL
