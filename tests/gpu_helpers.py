"""Helpers for the GPU parity tests: move seeded inputs to the device, run
libks through its C ABI, and compare with the fp64 oracle.

Comparison rules (the tolerance of the fp32 path):
* relative Frobenius error  ||Y - Y_ref||_F / ||Y_ref||_F  <= 1e-5 for fp32
  and for bf16 inputs (both sides use the same bf16 values, so only the fp32
  accumulation rounds; the looser 1e-2 budget for bf16 is never needed);
* elementwise, for single factors: |Y - Y_ref| <= c * 2^-23 * sum_gamma |K X|
  + tiny, the forward error bound of an fp32 sum of c exact-or-rounded
  products (rounding each product and each partial sum at most once),
  where the magnitude sum is the oracle applied to |K| and |X|;
* integer-valued inputs: exact equality.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from kronecker_sparse_structured_amd import datagen, libks

DEV = "cuda:0"
FP32_REL_TOL = 1e-5


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X visible to torch"


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        bits = datagen.bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_values(a: np.ndarray, bf16: bool):
    """fp64 copy of what the device sees (bf16-rounded if bf16)."""
    if bf16:
        return oracle.widen(datagen.bf16_bits(a), "bf16")
    return oracle.widen(a, "f32")


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    num = np.sum((y.astype(np.float64) - ref) ** 2)
    den = np.sum(ref ** 2)
    return float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))


def check_factor(p, X: np.ndarray, W: np.ndarray, Y: np.ndarray, bf16: bool = False,
                 w_bf16: bool | None = None, rows=None):
    """Compare device output Y (host copy, rows subset if `rows`) with the
    oracle on the same (rounded) inputs."""
    w_bf16 = bf16 if w_bf16 is None else w_bf16
    Xs = X if rows is None else X[rows]
    Xd = host_values(Xs, bf16)
    Wd = host_values(W, w_bf16)
    ref = oracle.ks_matmul(p, Wd, Xd)
    mag = oracle.ks_matmul(p, np.abs(Wd), np.abs(Xd))
    c = p[2]
    bound = c * 2.0 ** -23 * mag + 1e-30
    err = np.abs(Y.astype(np.float64) - ref)
    assert np.all(err <= bound), "elementwise bound exceeded: max ratio %g" % float(np.max(err / bound))
    e = rel_err(Y, ref)
    assert e <= FP32_REL_TOL, "relative Frobenius error %g" % e
    return e


def run_factor(p, Xt: torch.Tensor, Wt: torch.Tensor, kernel="auto", out=None, stream=None):
    return libks.matmul(Xt, Wt, p, out=out, kernel=kernel, stream=stream)


def sample_rows(batch: int, n: int = 48, seed: int = 7):
    """First and last rows plus a seeded random sample, sorted, unique."""
    rng = np.random.default_rng(seed)
    head = list(range(min(8, batch)))
    tail = list(range(max(0, batch - 8), batch))
    mid = list(rng.integers(0, batch, size=min(n, batch)))
    return np.array(sorted(set(head + tail + mid)), dtype=np.int64)


def chain_check(patterns, X: np.ndarray, Ws, Y: np.ndarray, bf16: bool, rows=None):
    Xs = X if rows is None else X[rows]
    Xd = host_values(Xs, bf16)
    Wd = [host_values(W, bf16) for W in Ws]
    se, sr, ma = oracle.ks_chain_err(patterns, Wd, Xd, Y)
    e = float(np.sqrt(se / sr))
    assert e <= FP32_REL_TOL, "relative Frobenius error %g (max abs %g)" % (e, ma)
    return e
