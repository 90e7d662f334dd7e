"""torch.autograd integration of the layer.

``moe_lora(x, logits, weights, dims)`` routes the tokens, runs the forward
and returns Y; its backward runs the library's backward and hands autograd
dX, the four LoRA-factor gradients and, when the logits require grad, the
logit gradient.  Only the LoRA factors train, so the base weights
must not require grad ("Faster LoRA MoE training").  The
factor gradients come out of the library in fp32; autograd casts each to
the dtype of the factor it belongs to (so a 16-bit copy of fp32 master
factors passes the fp32 values straight back through the cast).

Marshalling only: every step runs in the HIP library through the calls of
``api``; the routing, the saved forward buffers and the workspaces are
allocated per call by those wrappers.
"""
from __future__ import annotations

import torch

from . import api


class _MoELoRA(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, logits, w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down, dims):
        if ctx.needs_input_grad[2] or ctx.needs_input_grad[3]:
            raise ValueError("the base weights are frozen (only the LoRA factors train): "
                             "pass w_gate_up and w_down with requires_grad=False")
        weights = api.Weights(w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down)
        routing = api.route(logits, dims)
        y, saved = api.forward(x, routing, weights, dims)
        ctx.dims, ctx.routing, ctx.fwd_saved = dims, routing, saved
        ctx.save_for_backward(x, w_gate_up, w_down, a_gate_up, b_gate_up, a_down, b_down)
        return y

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, dy):
        x, *w = ctx.saved_tensors
        dims, need = ctx.dims, ctx.needs_input_grad
        router = api.empty_router_grads(dims, dy.device) if need[1] else None
        g = api.backward(dy.contiguous(), x, ctx.routing, api.Weights(*w), ctx.fwd_saved, dims,
                         router_out=router)
        ctx.routing = ctx.fwd_saved = None
        pick = lambda i, t: t if need[i] else None  # noqa: E731
        return (pick(0, g.dx), router.d_logits if router is not None else None, None, None,
                pick(4, g.da_gate_up), pick(5, g.db_gate_up), pick(6, g.da_down),
                pick(7, g.db_down), None)


def moe_lora(x: torch.Tensor, logits: torch.Tensor, weights: api.Weights,
             dims: api.Dims) -> torch.Tensor:
    """Y of the MoE-LoRA expert layer, differentiable in x, the logits and
    the four LoRA factors (inputs as for ``api.route`` / ``api.forward``:
    contiguous GPU tensors, x and the weights of the layer's element type,
    the logits fp32)."""
    return _MoELoRA.apply(x, logits, *weights, dims)
