"""ks_matmul_dw_noalloc (needs an MI355X): the dK entry point that allocates
nothing and keeps its partial sums in the library's scratch array, against
ks_matmul_dw (caller's workspace) and the fp64 oracle.

Two calls in a row on each pattern, the second with a smaller batch, so the
second runs over the scratch the first one left behind.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, FP32_REL_TOL, host_values, require_gpu, to_dev
from kronecker_sparse_structured_amd import libks

pytestmark = pytest.mark.gpu


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, dtype=np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def _dw_with_workspace(p, dY, X, batch, dt):
    a, b, c, d = p
    out = torch.full((a, d, b, c), float("nan"), dtype=torch.float32, device=DEV)
    nbytes = libks.ks_matmul_dw_workspace_size(p, batch, dt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV) if nbytes else None
    libks.ks_matmul_dw(p, dY, X, out, batch, dt, ws, nbytes)
    return out, nbytes


def _dw_noalloc(p, dY, X, batch, dt):
    a, b, c, d = p
    out = torch.full((a, d, b, c), float("nan"), dtype=torch.float32, device=DEV)
    libks.ks_matmul_dw_noalloc(p, dY, X, out, batch, dt)
    return out


# (pattern, first batch, second batch, bf16 X): matrix-core, small-block and
# generic dK kernels, each with partial sums in the scratch on the first call
CASES = [((4, 64, 16, 6), 25216, 3001, False), ((64, 8, 8, 8), 4096, 333, False),
         ((3, 5, 7, 2), 2000, 45, False), ((2, 128, 128, 4), 1024, 77, True),
         ((1, 16, 16, 4096), 512, 37, True), ((1, 32, 32, 128), 4096, 100, False)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%d_%d_%d_%d" % c[0])
def test_dw_noalloc_matches_workspace_entry_point(case):
    require_gpu()
    p, b1, b2, bf16 = case
    a, b, c, d = p
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    rng = np.random.default_rng(sum(p) + b1)
    X = rng.standard_normal((b1, a * c * d), dtype=np.float32)
    dY = rng.standard_normal((b1, a * b * d), dtype=np.float32)
    Xt, dYt = to_dev(X, bf16), to_dev(dY)
    print("case", p, b1, b2, "bf16" if bf16 else "f32", flush=True)
    for batch in (b1, b2):
        ref_dev, nbytes = _dw_with_workspace(p, dYt[:batch], Xt[:batch], batch, dt)
        got = _dw_noalloc(p, dYt[:batch], Xt[:batch], batch, dt)
        torch.cuda.synchronize()
        if batch == b1:
            assert nbytes > 0, "the first call should use partial sums"
        got_h, ref_h = got.cpu().numpy(), ref_dev.cpu().numpy()
        # the same kernels, row ranges and summation order: identical bits
        assert np.array_equal(got_h, ref_h), (p, batch)
        ref = oracle.ks_matmul_dw(p, host_values(dY[:batch], False), host_values(X[:batch], bf16))
        assert _rel(got_h, ref) <= FP32_REL_TOL, (p, batch)


def test_dw_noalloc_batch_zero_and_one():
    require_gpu()
    p = (4, 64, 16, 6)
    a, b, c, d = p
    out = torch.full((a, d, b, c), 5.0, device=DEV)
    libks.ks_matmul_dw_noalloc(p, None, None, out, 0, libks.DTYPE_F32)
    torch.cuda.synchronize()
    assert not out.any()
    rng = np.random.default_rng(3)
    X = rng.standard_normal((1, a * c * d), dtype=np.float32)
    dY = rng.standard_normal((1, a * b * d), dtype=np.float32)
    got = _dw_noalloc(p, to_dev(dY), to_dev(X), 1, libks.DTYPE_F32)
    torch.cuda.synchronize()
    ref = oracle.ks_matmul_dw(p, host_values(dY, False), host_values(X, False))
    assert _rel(got.cpu().numpy(), ref) <= FP32_REL_TOL
