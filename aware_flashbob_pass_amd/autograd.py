"""Softmax attention as a torch.autograd.Function whose backward is itself
differentiable, routed to the library's kernels at every order.

    O = softmax(tau Q K^T) V                 -> attn_fwd
    (dQ, dK, dV) = g(Q, K, V, dO)            -> attn_bwd
    J_g^T (UQ, UK, UV) = (gQ, gK, gV, gdO)   -> bob_attention_with_stats

so `torch.autograd.grad(loss, (q, k, v), create_graph=True)` followed by a
second `grad` (a Hessian-vector product, e.g. for Sophia-style Hessian
estimation) runs the exact backward-over-backward path on the GPU. This is the
attention-backend integration that the FlashBoB review page describes for
its end-to-end experiments (Summary; Weaknesses on the backend-integration
effect); the training loop itself is out of scope here.

The double-backward node returns the total derivative with respect to Q, K, V
and dO (the forward's O and row LSE L are functions of Q, K, V, so their
contributions are already inside gQ, gK, gV); it therefore takes O and L as
non-differentiable saved statistics.
"""

import math

import torch

from . import binding as _b


def _scale(tau, d):
    return float(1.0 / math.sqrt(d) if tau is None else tau)


class _AttentionBackward(torch.autograd.Function):
    """(Q, K, V, O, L, dO) -> (dQ, dK, dV); differentiable via BoB."""

    @staticmethod
    def forward(ctx, q, k, v, o, lse, do, tau, causal):
        do = do.contiguous()
        dq, dk, dv, dvec = _b.attn_bwd(q, k, v, o, do, lse, tau=tau, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse, dvec, do)
        ctx.tau, ctx.causal = tau, causal
        return dq, dk, dv

    @staticmethod
    def backward(ctx, uq, uk, uv):
        q, k, v, o, lse, dvec, do = ctx.saved_tensors
        zeros = None
        us = []
        for u in (uq, uk, uv):
            if u is None:
                if zeros is None:
                    zeros = torch.zeros_like(q)
                u = zeros
            us.append(u.contiguous())
        gq, gk, gv, gdo = _b.bob_attention_with_stats(q, k, v, do, us[0], us[1], us[2], o, lse, dvec,
                                                      tau=ctx.tau, causal=ctx.causal)
        return gq, gk, gv, None, None, gdo, None, None


class _Attention(torch.autograd.Function):
    """(Q, K, V) -> O with a differentiable backward."""

    @staticmethod
    def forward(ctx, q, k, v, tau, causal):
        o, lse = _b.attn_fwd(q, k, v, tau=tau, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.tau, ctx.causal = tau, causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _AttentionBackward.apply(q, k, v, o.detach(), lse.detach(), do, ctx.tau, ctx.causal)
        return dq, dk, dv, None, None


def attention(q, k, v, tau=None, causal=False):
    """Softmax attention over [B, H, N, d] GPU tensors with exact first and
    second derivatives from the library's kernels."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return _Attention.apply(q, k, v, _scale(tau, q.shape[-1]), bool(causal))
