"""torch.autograd functions over the C ABI: the GMA forward of each variant (bidirectional,
causal, cross-attention) with its backward (Sec. 4.1 of "Gaussian Mixture Attention").

Glue only: the forward calls gma_forward_*, the backward gma_backward_* of libgma.so; every
arithmetic step runs in the library's kernels.  Inputs are device tensors; X_Q, X_K, V share
one dtype (float32 or bfloat16), the mixture parameters are float32.  The gradients of the
parameters are float32, those of X_Q, X_K, V have the inputs' dtype.  No workspace is kept
between calls; each call asks the library for its size."""
from __future__ import annotations

import torch

from . import binding as gb

_KEYS = ("dXQ", "dXK", "dV", "dmu", "dsigma2", "dpi")


def _contiguous(*ts):
    return [t.contiguous() for t in ts]


class _GMA(torch.autograd.Function):
    @staticmethod
    def forward(ctx, variant, eps, chunk, xq, xk, v, mu, sigma2, pi):
        xq, xk, v, mu, sigma2, pi = _contiguous(xq, xk, v, mu, sigma2, pi)
        if variant == "bidir":
            out = gb.gma_forward_bidir(xq, xk, v, mu, sigma2, pi, eps)
        elif variant == "causal":
            out = gb.gma_forward_causal(xq, xk, v, mu, sigma2, pi, eps, chunk=chunk)
        else:
            out = gb.gma_forward_cross(xq, xk, v, mu, sigma2, pi, eps)
        ctx.save_for_backward(xq, xk, v, mu, sigma2, pi)
        ctx.variant, ctx.eps = variant, eps
        return out

    @staticmethod
    def backward(ctx, d_o):
        xq, xk, v, mu, sigma2, pi = ctx.saved_tensors
        fn = {"bidir": gb.gma_backward_bidir, "causal": gb.gma_backward_causal,
              "cross": gb.gma_backward_cross}[ctx.variant]
        g = fn(xq, xk, v, mu, sigma2, pi, d_o.to(xq.dtype).contiguous(), ctx.eps)
        return (None, None, None) + tuple(g[k] for k in _KEYS)


def gma_bidir(xq, xk, v, mu, sigma2, pi, eps: float = 1e-6) -> torch.Tensor:
    """Bidirectional GMA (Eq. 5-8), differentiable in every input."""
    return _GMA.apply("bidir", eps, 64, xq, xk, v, mu, sigma2, pi)


def gma_causal(xq, xk, v, mu, sigma2, pi, eps: float = 1e-6, chunk: int = 64) -> torch.Tensor:
    """Causal GMA (Eq. 6b, 8b), differentiable in every input."""
    return _GMA.apply("causal", eps, chunk, xq, xk, v, mu, sigma2, pi)


def gma_cross(xq, xk, v, mu, sigma2, pi, eps: float = 1e-6) -> torch.Tensor:
    """Cross-attention GMA (queries xq [B,H,N_q,d_r], context xk, v of N_k rows), differentiable
    in every input."""
    return _GMA.apply("cross", eps, 64, xq, xk, v, mu, sigma2, pi)
