"""torch.autograd wrappers of dispatch and combine (binding layer only).

Every forward and backward step runs in the library's kernels
(moe_layout + moe_dispatch, moe_combine, moe_combine_backward,
moe_dispatch_backward); these Functions only route tensors. Use one
MoeDispatcher(backward=True) per MoE layer: its persistent buffers hold that
layer's dispatched rows until the layer's next forward, and the small
per-call state the backward needs (row map, true total) is copied at forward
time so later layers cannot overwrite it.
"""
from __future__ import annotations

from typing import Optional

import torch

from .moe import MoeDispatcher


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, scores, ids, disp: MoeDispatcher, ntpr: int):
        lay = disp.layout(ids, ntpr)
        out = disp.dispatch(x, scores.detach(), ids, lay.counts, num_tokens_per_rank=ntpr)
        row_map = lay.row_map.clone()
        total = lay.offsets[-1:].clone()
        ctx.disp, ctx.T, ctx.ntpr, ctx.row_map = disp, x.shape[0], ntpr, row_map
        ctx.mark_non_differentiable(row_map, total)
        return out.x_e, row_map, total

    @staticmethod
    def backward(ctx, grad_x_e, _grad_row_map, _grad_total):
        g = grad_x_e.contiguous()
        grad_x = ctx.disp.dispatch_backward(g, ctx.row_map, ctx.T, num_tokens_per_rank=ctx.ntpr)
        return grad_x.clone(), None, None, None, None


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y_e, scores, row_map, total, disp: MoeDispatcher, ntpr: int):
        y = disp.combine(y_e, row_map, scores, num_tokens_per_rank=ntpr)
        ctx.save_for_backward(y_e, scores, row_map, total)
        ctx.disp, ctx.ntpr = disp, ntpr
        return y.clone()

    @staticmethod
    def backward(ctx, grad_y):
        y_e, scores, row_map, total = ctx.saved_tensors
        g_e, g_s = ctx.disp.combine_backward(grad_y.contiguous(), y_e, row_map, scores,
                                             num_tokens_per_rank=ctx.ntpr)
        # Rows past the true total did not reach y: their gradient is zero
        # (the buffer holds stale rows there).
        rows = torch.arange(y_e.shape[0], device=y_e.device)
        live = (rows < total)[:, None]
        grad_y_e = torch.where(live, g_e[: y_e.shape[0]], torch.zeros((), dtype=g_e.dtype,
                                                                       device=g_e.device))
        return grad_y_e, g_s.clone(), None, None, None, None


class MoeTokenDispatcher:
    """Differentiable dispatch/combine of one MoE layer.

        d = MoeTokenDispatcher(MoeDispatcher(nmax, D, E, K, backward=True))
        x_e = d.dispatch(x, scores, ids)        # [round_up4(ntpr) * K, D]
        y_e = experts(x_e)                      # rows [0, total) are the tokens'
        y = d.combine(y_e, scores)              # [T, D]
        y.backward(...)                         # dL/dx, dL/dscores, dL/dy_e
    """

    def __init__(self, dispatcher: MoeDispatcher):
        if not dispatcher.backward_enabled:
            raise ValueError("the MoeDispatcher needs backward=True")
        self.disp = dispatcher
        self._row_map: Optional[torch.Tensor] = None
        self._total: Optional[torch.Tensor] = None
        self._ntpr: Optional[int] = None

    def dispatch(self, x: torch.Tensor, topk_scores: torch.Tensor, topk_ids: torch.Tensor,
                 num_tokens_per_rank: Optional[int] = None) -> torch.Tensor:
        ntpr = x.shape[0] if num_tokens_per_rank is None else int(num_tokens_per_rank)
        x_e, self._row_map, self._total = _Dispatch.apply(
            x.contiguous(), topk_scores.contiguous(), topk_ids.contiguous(), self.disp, ntpr)
        self._ntpr = ntpr
        return x_e

    def combine(self, y_e: torch.Tensor, topk_scores: torch.Tensor) -> torch.Tensor:
        if self._row_map is None:
            raise RuntimeError("combine() needs a preceding dispatch() on this layer")
        return _Combine.apply(y_e.contiguous(), topk_scores.contiguous(), self._row_map,
                              self._total, self.disp, self._ntpr)
