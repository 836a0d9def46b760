"""torch.autograd binding of fa_fwd / fa_bwd (argument marshalling only: the
forward and the gradients are computed by libfa.so's kernels).

    out = varlen_attention(q, k, v, cfg, sink=None, alibi_slopes=None, drop_mask=None)

q [T_q, Nq, D], k, v [T_kv, Nkv, D] (or cfg's layout) require grad as needed; the
backward returns dQ, dK, dV (and dSink when a sink tensor requiring grad is given).
"""
from __future__ import annotations

import torch

from ._lib import Config, fa_bwd, fa_fwd


class _VarlenAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, sink, cfg: Config, alibi_slopes, drop_mask):
        q, k, v = q.detach(), k.detach(), v.detach()
        sink_d = None if sink is None else sink.detach()
        out, m, l = fa_fwd(cfg, q, k, v, drop_mask, alibi_slopes, sink_d)
        ctx.cfg = cfg
        ctx.extra = (alibi_slopes, drop_mask)
        ctx.save_for_backward(q, k, v, out, m, l, sink_d if sink_d is not None else torch.empty(0))
        ctx.has_sink = sink is not None
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, m, l, sink = ctx.saved_tensors
        alibi_slopes, drop_mask = ctx.extra
        dq, dk, dv, dsink = fa_bwd(ctx.cfg, q, k, v, dout.contiguous(), out, m, l, drop_mask, alibi_slopes,
                                   sink if ctx.has_sink else None)
        return dq, dk, dv, (dsink if ctx.has_sink else None), None, None, None


def varlen_attention(q, k, v, cfg: Config, sink=None, alibi_slopes=None, drop_mask=None):
    """Attention output of fa_fwd with gradients from fa_bwd (see include/fa.h for the arguments)."""
    return _VarlenAttention.apply(q, k, v, sink, cfg, alibi_slopes, drop_mask)
