"""torch.autograd wrapper of the operator: the forward runs prism_fwd_ckpt where
the chunkwise backward serves the shape (keeping every chunk's start state for
the backward, prism_bwd_ckpt, which stores the token-sized gradients of bf16
inputs in bf16 directly), else prism_fwd_resume and prism_bwd_ex (all in
libprism; nothing is computed here except casting the remaining fp32 gradients
to each input's dtype).

    o, S_final = prism(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L,
                       S_init=None, residual="linear")

Gradients flow to q, k, v, u, g, b, a, h, conv_w and S_init (fp32), for the
upstream gradients of o and S_final (either may be unused).  The carried
convolution history of prism_fwd_resume is not taken: the backward entry point
differentiates sequences that start with a zero history.
"""
from __future__ import annotations

import torch

from . import binding

_INPUTS = ("q", "k", "v", "u", "g", "b", "a", "h", "conv_w")


class PrismFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, S_init, residual):
        ckpt = None
        if binding.checkpoint_bytes(binding._dims_of(q, v, cu_seqlens)) > 0:
            try:
                o, S_final, ckpt = binding.fwd_ckpt(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L,
                                                    S_init=S_init, residual=residual)
            except binding.PrismError as err:        # the environment selects another scan
                if err.status != binding.PRISM_EUNSUPPORTED:
                    raise
        if ckpt is None:
            o, S_final, _ = binding.fwd_resume(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L,
                                               S_init=S_init, residual=residual)
        ctx.save_for_backward(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, S_init, ckpt)
        ctx.L, ctx.residual = L, residual
        ctx.has_s_init = S_init is not None
        return o, S_final

    @staticmethod
    def backward(ctx, d_o, d_s):
        q, k, v, u, g, b, a, h, conv_w, cu_seqlens, S_init, ckpt = ctx.saved_tensors
        if not ctx.has_s_init:
            S_init = None
        d_o = torch.zeros_like(v) if d_o is None else d_o.to(v.dtype).contiguous()
        d_s = None if d_s is None else d_s.to(torch.float32).contiguous()
        want_s = ctx.has_s_init and ctx.needs_input_grad[11]
        args = (q, k, v, u, g, b, a, h, conv_w, cu_seqlens, ctx.L, d_o)
        kw = dict(dS_final=d_s, S_init=S_init, want_dS_init=want_s, residual=ctx.residual)
        grads = None
        if ckpt is not None:
            try:
                gdt = torch.bfloat16 if q.dtype == torch.bfloat16 else None
                grads = binding.bwd(*args, checkpoints=ckpt, grad_dtype=gdt, **kw)
            except binding.PrismError as err:        # PRISM_BWD_CHUNKED=0 since the forward
                if err.status != binding.PRISM_EUNSUPPORTED:
                    raise
        if grads is None:
            grads = binding.bwd(*args, **kw)
        src = dict(zip(_INPUTS, (q, k, v, u, g, b, a, h, conv_w)))
        out = []
        for i, name in enumerate(_INPUTS):
            gr = grads[name]
            out.append(None if gr is None or not ctx.needs_input_grad[i] else gr.to(src[name].dtype))
        return (*out, None, None, grads["S_init"] if want_s else None, None)


def prism(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, S_init=None, residual="linear"):
    """Differentiable forward pass: returns (o, S_final)."""
    return PrismFunction.apply(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, S_init, residual)
