"""KSLinear: a chain of KS factors as a PyTorch layer, forward and backward
through libks (KS abstract page, taxoreview.com "dblp:303/4794", first
paragraph: the layer built from KS factors; the gradients are the chain rule
on Y = X W^T, see include/ks.h).

Argument marshalling only: every product runs in the HIP library. With
gradients enabled each factor is its own launch, so that the intermediates
the backward pass needs are kept; without, the chain goes through
``chain_matmul`` and may run fused pairs.
"""
from __future__ import annotations

import math
from typing import Sequence

from . import libks


def _autograd():
    import torch

    class KSMatmulFunction(torch.autograd.Function):
        """Y = X W^T for one factor; dX = dY W and dK through libks."""

        @staticmethod
        def forward(ctx, X, W, pattern):
            ctx.pattern = tuple(int(v) for v in pattern)
            ctx.save_for_backward(X, W)
            return libks.matmul(X, W, ctx.pattern)

        @staticmethod
        def backward(ctx, dY):
            X, W = ctx.saved_tensors
            dY = dY.contiguous()
            if dY.dtype != torch.float32:
                dY = dY.float()
            dX = dW = None
            if ctx.needs_input_grad[0]:
                dX = libks.matmul_dx(dY, W, ctx.pattern).to(X.dtype)
            if ctx.needs_input_grad[1]:
                dW = libks.matmul_dw(dY, X, ctx.pattern).to(W.dtype)
            return dX, dW, None

    return KSMatmulFunction


_FN = None


def ks_matmul_autograd(X, W, pattern):
    """Differentiable Y = X W^T for one KS factor (X: (batch, a*c*d))."""
    global _FN
    if _FN is None:
        _FN = _autograd()
    return _FN.apply(X, W, pattern)


def make_layer_class():
    import torch

    class KSLinear(torch.nn.Module):
        """y = x (W_{L-1} ... W_0)^T for KS factors p[0], ..., p[L-1] (applied
        in that order); weights K_k of shape (a, d, b, c), initialised
        N(0, 1/c). Input (..., n_in); output (..., n_out), fp32."""

        def __init__(self, patterns: Sequence[Sequence[int]], dtype=None, device=None, seed: int = 0):
            super().__init__()
            self.patterns = [tuple(int(v) for v in p) for p in patterns]
            for k in range(1, len(self.patterns)):
                a0, b0, _, d0 = self.patterns[k - 1]
                a1, _, c1, d1 = self.patterns[k]
                if a0 * b0 * d0 != a1 * c1 * d1:
                    raise ValueError("factor %d output width does not match factor %d input" % (k - 1, k))
            gen = torch.Generator(device="cpu").manual_seed(seed)
            ws = []
            for (a, b, c, d) in self.patterns:
                w = torch.randn((a, d, b, c), generator=gen) / math.sqrt(c)
                ws.append(torch.nn.Parameter(w.to(device=device, dtype=dtype or torch.float32)))
            self.weights = torch.nn.ParameterList(ws)

        @property
        def n_in(self):
            a, _, c, d = self.patterns[0]
            return a * c * d

        @property
        def n_out(self):
            a, b, _, d = self.patterns[-1]
            return a * b * d

        def forward(self, x):
            lead = x.shape[:-1]
            x2 = x.reshape(-1, self.n_in).contiguous()
            grad = torch.is_grad_enabled() and (x.requires_grad or any(w.requires_grad for w in self.weights))
            same = all(w.dtype == x2.dtype for w in self.weights) and x2.dtype in (torch.float32, torch.bfloat16)
            if not grad and same:
                y = libks.chain_matmul(x2, list(self.weights), self.patterns)
            else:
                y = x2
                for p, w in zip(self.patterns, self.weights):
                    if not (y.dtype == w.dtype or y.dtype == torch.float32):
                        y = y.float()
                    y = ks_matmul_autograd(y, w, p) if grad else libks.matmul(y, w, p)
            return y.reshape(*lead, self.n_out)

    return KSLinear


_LAYER = None


def __getattr__(name):
    """``layer.KSLinear`` builds the class on first use (torch is imported
    lazily, as everywhere in this package)."""
    global _LAYER
    if name == "KSLinear":
        if _LAYER is None:
            _LAYER = make_layer_class()
        return _LAYER
    raise AttributeError(name)
