"""Checks that pin the fp64 oracle to facts that do not come from the oracle.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with an independent source:

* the Kronecker definition evaluated by ``numpy.kron`` (KS abstract page,
  taxoreview.com "dblp:303/4794", first paragraph: supports are Kronecker
  products of identity and all-ones blocks);
* textbook reductions: a = d = 1 is a dense GEMM, d = 1 is block diagonal
  (``scipy.linalg.block_diag``);
* the Sylvester-Hadamard closed form for butterfly chains with
  [[1, 1], [1, -1]] blocks (``scipy.linalg.hadamard`` and
  (-1)^popcount(i & j)); butterfly supports are named on the same page,
  third paragraph;
* the permute / batched-multiply / permute formulation the abstract ascribes
  to existing kernels (second sentence), via ``numpy.einsum``;
* hand-derived worked examples in ``tests/golden/ks_worked_examples.json``;
* one-hot and NaN-propagation probes, linearity and the adjoint identity.

Integer-valued data keeps every sum exact, so most pins compare for exact
equality. The same functions run against deliberately broken oracle builds
in ``test_oracle_mutants.py`` to show that each plausible mistake is caught.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "ks_worked_examples.json")


def dense_from_kron(p, K):
    """Dense W = sum over (alpha, delta) of E_alpha (x) K[alpha, delta] (x) E_delta,
    where E_i is the matrix unit at (i, i): a matrix whose support lies in
    I_a (x) 1_{b x c} (x) I_d, built with numpy.kron."""
    a, b, c, d = p
    W = np.zeros((a * b * d, a * c * d))
    for al in range(a):
        Ea = np.zeros((a, a))
        Ea[al, al] = 1.0
        for de in range(d):
            Ed = np.zeros((d, d))
            Ed[de, de] = 1.0
            W += np.kron(np.kron(Ea, K[al, de].astype(np.float64)), Ed)
    return W


def support_mask(p):
    a, b, c, d = p
    return np.kron(np.kron(np.eye(a), np.ones((b, c))), np.eye(d))


def int_data(rng, shape):
    return rng.integers(-8, 9, size=shape).astype(np.float64)


def small_patterns():
    return list(itertools.product([1, 2, 3, 4], repeat=4))


def pin_dense_kron_brute_force(lib, patterns=None, batches=(1, 5)):
    """Every pattern with a, b, c, d in {1..4} (plus a few wider ones): the
    oracle equals X @ W^T with W from numpy.kron, exactly, on integer data."""
    rng = np.random.default_rng(101)
    pats = patterns if patterns is not None else small_patterns() + [
        (3, 2, 5, 2), (2, 4, 4, 2), (4, 64, 16, 6), (1, 3, 7, 5)]
    for p in pats:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        W = dense_from_kron(p, K)
        assert np.array_equal(W != 0, (W != 0) & (support_mask(p) != 0)), p
        for B in batches:
            X = int_data(rng, (B, a * c * d))
            Y = oracle.ks_matmul(p, K, X, lib=lib)
            assert np.array_equal(Y, X @ W.T), (p, B)


def pin_support_is_kronecker_mask(lib):
    """With all-nonzero weights, the oracle's dependency pattern (one-hot
    columns) is exactly I_a (x) 1_{b x c} (x) I_d."""
    for p in [(2, 3, 2, 2), (1, 4, 4, 3), (3, 1, 2, 4), (2, 2, 3, 1)]:
        a, b, c, d = p
        K = np.arange(1, a * b * c * d + 1, dtype=np.float64).reshape(a, d, b, c)
        X = np.eye(a * c * d)
        Y = oracle.ks_matmul(p, K, X, lib=lib)      # row j = column j of W
        assert np.array_equal(Y.T != 0, support_mask(p) != 0), p
        assert np.array_equal(Y.T, dense_from_kron(p, K)), p


def pin_dense_gemm_a1_d1(lib):
    """a = d = 1: Y = X @ K[0, 0]^T (numpy matmul), fp64 random data."""
    rng = np.random.default_rng(102)
    for b, c in [(1, 1), (3, 5), (16, 16), (64, 16), (7, 128)]:
        K = rng.standard_normal((1, 1, b, c))
        X = rng.standard_normal((9, c))
        Y = oracle.ks_matmul((1, b, c, 1), K, X, lib=lib)
        np.testing.assert_allclose(Y, X @ K[0, 0].T, rtol=1e-13, atol=1e-13)


def pin_block_diagonal_d1(lib):
    """d = 1: W is block diagonal with blocks K[alpha, 0]."""
    rng = np.random.default_rng(103)
    for a, b, c in [(2, 3, 2), (4, 4, 4), (5, 1, 3), (3, 2, 6)]:
        K = int_data(rng, (a, 1, b, c))
        W = scipy.linalg.block_diag(*[K[al, 0] for al in range(a)])
        X = int_data(rng, (6, a * c))
        Y = oracle.ks_matmul((a, b, c, 1), K, X, lib=lib)
        assert np.array_equal(Y, X @ W.T), (a, b, c)


def pin_diagonal(lib):
    """a = 1, b = c = 1: W = diag(K[0, :, 0, 0])."""
    rng = np.random.default_rng(104)
    for d in [1, 2, 7]:
        K = int_data(rng, (1, d, 1, 1))
        X = int_data(rng, (4, d))
        Y = oracle.ks_matmul((1, 1, 1, d), K, X, lib=lib)
        assert np.array_equal(Y, X * K[0, :, 0, 0][None, :]), d


def hadamard_chain(L):
    pats = [(2 ** k, 2, 2, 2 ** (L - 1 - k)) for k in range(L)]
    Ks = []
    for (a, b, c, d) in pats:
        K = np.empty((a, d, 2, 2))
        K[...] = np.array([[1.0, 1.0], [1.0, -1.0]])
        Ks.append(K)
    return pats, Ks


def pin_hadamard(lib):
    """The chain of (2^k, 2, 2, 2^(L-1-k)) factors with [[1,1],[1,-1]] blocks
    maps X to X H, H the 2^L Sylvester-Hadamard matrix; applying it twice
    gives 2^L X. Exact in integers."""
    rng = np.random.default_rng(105)
    for L in [1, 2, 3, 4, 5, 6]:
        n = 2 ** L
        pats, Ks = hadamard_chain(L)
        H = scipy.linalg.hadamard(n).astype(np.float64)
        i = np.arange(n)
        Hc = np.array([[(-1.0) ** bin(x & y).count("1") for y in i] for x in i])
        assert np.array_equal(H, Hc)
        X = rng.integers(-8, 9, size=(5, n)).astype(np.float64)
        Y = oracle.ks_chain_matmul(pats, Ks, X, lib=lib)
        assert np.array_equal(Y, X @ H), L
        Y2 = oracle.ks_chain_matmul(pats + pats, Ks + Ks, X, lib=lib)
        assert np.array_equal(Y2, n * X), L


def pin_worked_examples(lib):
    """Hand-derived fixtures in tests/golden/ks_worked_examples.json."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        p = tuple(case["pattern"])
        a, b, c, d = p
        K = np.array(case["K"], dtype=np.float64).reshape(a, d, b, c)
        X = np.array(case["X"], dtype=np.float64)
        Y = oracle.ks_matmul(p, K, X, lib=lib)
        assert np.array_equal(Y, np.array(case["Y"], dtype=np.float64)), case["name"]
        assert np.array_equal(dense_from_kron(p, K), np.array(case["W"], dtype=np.float64)), case["name"]


def pin_nan_support(lib):
    """A NaN at input (alpha, gamma, delta) poisons exactly the outputs
    (alpha, all beta, delta)."""
    rng = np.random.default_rng(106)
    for p in [(3, 2, 4, 5), (2, 5, 3, 1), (1, 3, 3, 4)]:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        K[K == 0] = 1.0
        for (al, ga, de) in [(0, 0, 0), (a - 1, c - 1, d - 1), (a // 2, c // 2, d // 2)]:
            X = int_data(rng, (2, a * c * d))
            X[0, (al * c + ga) * d + de] = np.nan
            Y = oracle.ks_matmul(p, K, X, lib=lib)
            bad = np.isnan(Y[0]).reshape(a, b, d)
            expect = np.zeros((a, b, d), dtype=bool)
            expect[al, :, de] = True
            assert np.array_equal(bad, expect), (p, al, ga, de)
            assert not np.isnan(Y[1]).any()


def pin_einsum_permutation_form(lib):
    """Permute X to (alpha, delta) batches of c-vectors, multiply by the b x c
    blocks, permute back: numpy.einsum('nacd,adbc->nabd')."""
    rng = np.random.default_rng(107)
    for p in [(2, 3, 4, 5), (4, 64, 16, 6), (3, 2, 2, 1), (1, 8, 8, 8), (5, 1, 2, 3)]:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        X = int_data(rng, (7, a * c * d))
        ref = np.einsum("nacd,adbc->nabd", X.reshape(7, a, c, d), K).reshape(7, a * b * d)
        assert np.array_equal(oracle.ks_matmul(p, K, X, lib=lib), ref), p


def pin_linearity_and_adjoint(lib):
    """f(X1 + X2) = f(X1) + f(X2), and <f_p(X), Z> = <X, f_p'(Z)> with
    p' = (a, c, b, d) and each block transposed (W^T is again KS)."""
    rng = np.random.default_rng(108)
    for p in [(2, 3, 4, 5), (3, 5, 2, 2), (1, 4, 6, 3), (4, 2, 2, 1)]:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        X1 = int_data(rng, (3, a * c * d))
        X2 = int_data(rng, (3, a * c * d))
        f = lambda X: oracle.ks_matmul(p, K, X, lib=lib)
        assert np.array_equal(f(X1 + X2), f(X1) + f(X2)), p
        Z = int_data(rng, (3, a * b * d))
        Kt = np.ascontiguousarray(K.transpose(0, 1, 3, 2))
        lhs = np.sum(f(X1) * Z)
        rhs = np.sum(X1 * oracle.ks_matmul((a, c, b, d), Kt, Z, lib=lib))
        assert lhs == rhs, p


def pin_chain_dense_product(lib):
    """A chain equals X @ (W_{L-1} ... W_0)^T with dense factors from
    numpy.kron; the order matters (random factors do not commute)."""
    rng = np.random.default_rng(109)
    chains = [
        [(1, 4, 2, 4), (4, 2, 2, 2)],          # 8 -> 16 -> 16
        [(2, 2, 2, 2), (1, 2, 2, 4), (4, 2, 2, 1)],
        [(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)],  # 6 -> 18 -> 12 -> 8
    ]
    for pats in chains:
        Ks = [int_data(rng, (a, d, b, c)) for (a, b, c, d) in pats]
        M = np.eye(pats[0][0] * pats[0][2] * pats[0][3])
        for p, K in zip(pats, Ks):
            M = dense_from_kron(p, K) @ M
        X = int_data(rng, (4, M.shape[1]))
        assert np.array_equal(oracle.ks_chain_matmul(pats, Ks, X, lib=lib), X @ M.T), pats
    # order: two square factors that do not commute
    p0, p1 = (1, 2, 2, 4), (4, 2, 2, 1)
    K0, K1 = int_data(rng, (1, 4, 2, 2)), int_data(rng, (4, 1, 2, 2))
    X = int_data(rng, (3, 8))
    fwd = oracle.ks_chain_matmul([p0, p1], [K0, K1], X, lib=lib)
    rev = oracle.ks_chain_matmul([p1, p0], [K1, K0], X, lib=lib)
    W0, W1 = dense_from_kron(p0, K0), dense_from_kron(p1, K1)
    assert np.array_equal(fwd, X @ (W1 @ W0).T)
    assert np.array_equal(rev, X @ (W0 @ W1).T)
    assert not np.array_equal(fwd, rev)


def pin_chain_err_streaming(lib):
    """The streaming error routine agrees with an explicit comparison."""
    rng = np.random.default_rng(110)
    pats = [(2, 3, 2, 2), (3, 2, 4, 1)]
    Ks = [rng.standard_normal((a, d, b, c)) for (a, b, c, d) in pats]
    X = rng.standard_normal((6, 8))
    ref = oracle.ks_chain_matmul(pats, Ks, X, lib=lib)
    cand = (ref + 1e-3 * rng.standard_normal(ref.shape)).astype(np.float32)
    se, sr, ma = oracle.ks_chain_err(pats, Ks, X, cand, lib=lib)
    diff = cand.astype(np.float64) - ref
    np.testing.assert_allclose(se, np.sum(diff ** 2), rtol=1e-12)
    np.testing.assert_allclose(sr, np.sum(ref ** 2), rtol=1e-12)
    np.testing.assert_allclose(ma, np.max(np.abs(diff)), rtol=1e-12)


def pin_backward_dense(lib):
    """Gradients of Y = X W^T against the dense W from numpy.kron: dX equals
    dY @ W, and dK equals dY^T @ X read at each K entry's position in W
    (row alpha*b*d + beta*d + delta, column alpha*c*d + gamma*d + delta), on
    integer data, exactly. Also a = d = 1 (dense GEMM gradients) and batch 0
    (dK = 0)."""
    rng = np.random.default_rng(111)
    pats = [(2, 3, 4, 5), (3, 5, 2, 2), (1, 4, 6, 3), (4, 2, 2, 1), (1, 7, 5, 1), (2, 1, 3, 4), (3, 2, 1, 2)]
    for p in pats:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        X = int_data(rng, (6, a * c * d))
        dY = int_data(rng, (6, a * b * d))
        W = dense_from_kron(p, K)
        assert np.array_equal(oracle.ks_matmul_dx(p, K, dY, lib=lib), dY @ W), p
        G = dY.T @ X
        ref = np.empty((a, d, b, c))
        for al, de, be, ga in itertools.product(range(a), range(d), range(b), range(c)):
            ref[al, de, be, ga] = G[al * b * d + be * d + de, al * c * d + ga * d + de]
        assert np.array_equal(oracle.ks_matmul_dw(p, dY, X, lib=lib), ref), p
    A, B = int_data(rng, (5, 4)), int_data(rng, (5, 3))     # a = d = 1: Y = X K^T with K (3 x 4)
    K = int_data(rng, (1, 1, 3, 4))
    assert np.array_equal(oracle.ks_matmul_dx((1, 3, 4, 1), K, B, lib=lib), B @ K[0, 0])
    assert np.array_equal(oracle.ks_matmul_dw((1, 3, 4, 1), B, A, lib=lib)[0, 0], B.T @ A)
    z = oracle.ks_matmul_dw((2, 3, 4, 5), np.zeros((0, 30)), np.zeros((0, 40)), lib=lib)
    assert z.shape == (2, 5, 3, 4) and not z.any()


def pin_backward_adjoint(lib):
    """<dY, f(X)> = <dL/dX, X> = <dL/dK, K> for L = <dY, f(X)> with f linear
    in both X and K; and the gradient in X is the forward map of the
    transposed pattern (a, c, b, d) with transposed blocks."""
    rng = np.random.default_rng(112)
    for p in [(2, 3, 4, 5), (1, 6, 2, 3), (5, 2, 3, 1), (3, 4, 4, 2)]:
        a, b, c, d = p
        K = int_data(rng, (a, d, b, c))
        X = int_data(rng, (4, a * c * d))
        dY = int_data(rng, (4, a * b * d))
        L = np.sum(dY * oracle.ks_matmul(p, K, X, lib=lib))
        dX = oracle.ks_matmul_dx(p, K, dY, lib=lib)
        dK = oracle.ks_matmul_dw(p, dY, X, lib=lib)
        assert np.sum(dX * X) == L, p
        assert np.sum(dK * K) == L, p
        Kt = np.ascontiguousarray(K.transpose(0, 1, 3, 2))
        assert np.array_equal(dX, oracle.ks_matmul((a, c, b, d), Kt, dY, lib=lib)), p


ALL_PINS = [
    pin_dense_kron_brute_force,
    pin_support_is_kronecker_mask,
    pin_dense_gemm_a1_d1,
    pin_block_diagonal_d1,
    pin_diagonal,
    pin_hadamard,
    pin_worked_examples,
    pin_nan_support,
    pin_einsum_permutation_form,
    pin_linearity_and_adjoint,
    pin_chain_dense_product,
    pin_chain_err_streaming,
    pin_backward_dense,
    pin_backward_adjoint,
]
