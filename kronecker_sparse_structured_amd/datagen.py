"""Seeded synthetic inputs for KS matrix multiplication.

This module is shared by the tests, the benchmark, the HIP path and the
oracle's callers. It holds no KS arithmetic: it only draws random numbers,
rounds fp32 draws to bf16 bit patterns, and names the workloads.

Recipe (one NumPy PCG64 generator per workload, ``default_rng(seed)``):
  1. X is drawn first, row-major, ``standard_normal(dtype=float32)`` (or
     integers uniform on [-8, 8] for the Hadamard check, stored as fp32);
  2. then the factor weights W_0 ... W_{L-1}, each of shape (a, d, b, c),
     ``standard_normal(dtype=float32)`` multiplied by sigma in fp32;
     sigma is a standard deviation;
  3. bf16 inputs are the round-to-nearest-even images of those fp32 draws.

Workload shapes mirror the layers the KS abstract page (taxoreview.com
"dblp:303/4794", last sentence) evaluates end to end: a ViT-S/16 MLP
up-projection (384 -> 1536 over 128 images x 197 tokens), a GPT-2-medium MLP
(1024 -> 4096 over 16 sequences x 1024 tokens), a square n = 4096 sweep over
KS patterns, and a four-factor butterfly at n = 65,536. The pages give no
pattern list or batch sizes; these synthetic shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

Pattern = Tuple[int, int, int, int]


def n_in(p: Sequence[int]) -> int:
    a, b, c, d = p
    return a * c * d


def n_out(p: Sequence[int]) -> int:
    a, b, c, d = p
    return a * b * d


def nnz(p: Sequence[int]) -> int:
    a, b, c, d = p
    return a * b * c * d


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.
    NaN maps to a quiet NaN with the same sign; infinities are kept."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)
    return r


@dataclass
class Workload:
    """A named KS workload: factors applied in order to a batch of rows."""
    name: str
    patterns: List[Pattern]
    batch: int
    sigmas: List[float]
    seed: int
    x_kind: str = "normal"      # "normal" (N(0,1)) or "int8range" (integers in [-8, 8])
    w_kind: str = "normal"      # "normal" (N(0, sigma)) or "hadamard" ([[1,1],[1,-1]] blocks)
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_in(self) -> int:
        return n_in(self.patterns[0])

    @property
    def n_out(self) -> int:
        return n_out(self.patterns[-1])


def hadamard_patterns(L: int) -> List[Pattern]:
    """Factors (2^k, 2, 2, 2^(L-1-k)) for k = 0..L-1."""
    return [(2 ** k, 2, 2, 2 ** (L - 1 - k)) for k in range(L)]


def square_sweep_patterns(n: int = 4096, sizes=(4, 8, 16, 32, 64, 128)) -> List[Pattern]:
    """Every (a, b, b, d) with b in sizes, a*b*d = n, a and d powers of two;
    ordered b ascending, then a ascending."""
    out: List[Pattern] = []
    for b in sizes:
        a = 1
        while a * b <= n:
            d = n // (a * b)
            out.append((a, b, b, d))
            a *= 2
    return out


def workloads() -> dict:
    """The five workload families, by name."""
    w = {}
    w["tiny"] = Workload("tiny", [(2, 4, 4, 2)], 32, [1.0], 1,
                         note="single factor, W 16x16 with 64 nonzeros")
    w["hadamard16"] = Workload("hadamard16", hadamard_patterns(4), 32, [1.0] * 4, 11,
                               x_kind="int8range", w_kind="hadamard",
                               note="product of the four factors is the 16x16 Walsh-Hadamard matrix")
    w["vit_mlp"] = Workload("vit_mlp", [(4, 64, 16, 6)], 25216, [1.0 / np.sqrt(16.0)], 2,
                            note="ViT-S/16 MLP up-projection 384->1536, 128 images x 197 tokens")
    w["gpt2_mlp"] = Workload("gpt2_mlp", [(1, 64, 16, 64), (64, 8, 8, 8)], 16384,
                             [1.0 / np.sqrt(16.0), 1.0 / np.sqrt(8.0)], 4,
                             note="GPT-2-medium MLP 1024->4096 as two KS factors, 16 seqs x 1024 tokens")
    w["butterfly65536"] = Workload("butterfly65536", [(16 ** k, 16, 16, 16 ** (3 - k)) for k in range(4)],
                                   4096, [0.25] * 4, 5,
                                   note="four butterfly factors at n = 65,536")
    # deep chains of small blocks (one row-resident launch when fused)
    w["radix2_n1024"] = Workload("radix2_n1024", [(2 ** k, 2, 2, 2 ** (9 - k)) for k in range(10)], 16384,
                                 [1.0 / np.sqrt(2.0)] * 10, 6,
                                 note="radix-2 butterfly, ten factors at n = 1024")
    w["radix4_n4096"] = Workload("radix4_n4096", [(4 ** k, 4, 4, 4 ** (5 - k)) for k in range(6)], 16384,
                                 [0.5] * 6, 7,
                                 note="radix-4 butterfly, six factors at n = 4096")
    w["radix8_n4096"] = Workload("radix8_n4096", [(8 ** k, 8, 8, 8 ** (3 - k)) for k in range(4)], 16384,
                                 [1.0 / np.sqrt(8.0)] * 4, 8,
                                 note="radix-8 butterfly, four factors at n = 4096")
    # butterflies on rows wider than LDS holds: runs of factors cut by slab
    # (common divisor of the a's) and index class (common divisor of the d's)
    w["radix2_n65536"] = Workload("radix2_n65536", [(2 ** k, 2, 2, 2 ** (15 - k)) for k in range(16)], 4096,
                                  [1.0 / np.sqrt(2.0)] * 16, 12,
                                  note="radix-2 butterfly, sixteen factors at n = 65,536")
    w["radix4_n65536"] = Workload("radix4_n65536", [(4 ** k, 4, 4, 4 ** (7 - k)) for k in range(8)], 4096,
                                  [0.5] * 8, 13,
                                  note="radix-4 butterfly, eight factors at n = 65,536")
    w["radix2_n16384"] = Workload("radix2_n16384", [(2 ** k, 2, 2, 2 ** (13 - k)) for k in range(14)], 16384,
                                  [1.0 / np.sqrt(2.0)] * 14, 14,
                                  note="radix-2 butterfly, fourteen factors at n = 16,384")
    # a radix-16 pair the strided-pair kernel fuses (e = 4): (64, 16, 16, 64)
    # then (1024, 16, 16, 4) at n = 65,536 (not a configuration of the pages)
    w["strided_pair_e4"] = Workload("strided_pair_e4", [(64, 16, 16, 64), (1024, 16, 16, 4)], 4096, [0.25] * 2, 9,
                                    note="two radix-16 factors four elements apart, n = 65,536")
    # a Monarch-shaped pair: 32 blocks of 32 x 32, then the mixing factor
    # across blocks, at n = 1024 (Monarch matrices as KS chains; the pages
    # give no sizes, so these are synthetic)
    w["monarch_n1024"] = Workload("monarch_n1024", [(32, 32, 32, 1), (1, 32, 32, 32)], 65536,
                                  [1.0 / np.sqrt(32.0)] * 2, 10,
                                  note="Monarch pair, 32 blocks of 32 x 32 then their mixing, n = 1024")
    for p_idx, p in enumerate(square_sweep_patterns()):
        name = "square_%d_%d_%d_%d" % p
        w[name] = Workload(name, [p], 16384, [1.0 / np.sqrt(p[2])], 3000 + p_idx,
                           note="square n=4096 sweep, pattern index %d" % p_idx)
    return w


def get(name: str) -> Workload:
    return workloads()[name]


def scaled(wl: Workload, batch: int) -> Workload:
    """The same workload with another batch size (same seed and draw order)."""
    return Workload(wl.name, list(wl.patterns), batch, list(wl.sigmas), wl.seed,
                    wl.x_kind, wl.w_kind, wl.note, dict(wl.extra))


def draw(wl: Workload):
    """Draw (X, [W_0, ..., W_{L-1}]) as fp32 NumPy arrays in the recipe order.
    X has shape (batch, n_in); W_k has shape (a, d, b, c)."""
    rng = np.random.default_rng(wl.seed)
    if wl.x_kind == "normal":
        X = rng.standard_normal((wl.batch, wl.n_in), dtype=np.float32)
    elif wl.x_kind == "int8range":
        X = rng.integers(-8, 9, size=(wl.batch, wl.n_in)).astype(np.float32)
    else:
        raise ValueError(wl.x_kind)
    Ws = []
    for p, s in zip(wl.patterns, wl.sigmas):
        a, b, c, d = p
        if wl.w_kind == "normal":
            W = rng.standard_normal((a, d, b, c), dtype=np.float32) * np.float32(s)
        elif wl.w_kind == "hadamard":
            if (b, c) != (2, 2):
                raise ValueError("hadamard blocks need b = c = 2")
            W = np.empty((a, d, 2, 2), dtype=np.float32)
            W[...] = np.array([[1.0, 1.0], [1.0, -1.0]], dtype=np.float32)
        else:
            raise ValueError(wl.w_kind)
        Ws.append(np.ascontiguousarray(W, dtype=np.float32))
    return X, Ws


def random_pattern_inputs(p: Pattern, batch: int, seed: int, kind: str = "normal"):
    """X (batch x a*c*d) and W (a, d, b, c) for ad-hoc test patterns."""
    rng = np.random.default_rng(seed)
    a, b, c, d = p
    if kind == "normal":
        X = rng.standard_normal((batch, a * c * d), dtype=np.float32)
        W = rng.standard_normal((a, d, b, c), dtype=np.float32) * np.float32(1.0 / np.sqrt(c))
    elif kind == "int8range":
        X = rng.integers(-8, 9, size=(batch, a * c * d)).astype(np.float32)
        W = rng.integers(-8, 9, size=(a, d, b, c)).astype(np.float32)
    else:
        raise ValueError(kind)
    return X, W
