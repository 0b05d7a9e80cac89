"""torch.autograd wrappers of dispatch and combine (binding layer only).

Every forward and backward step runs in the library's kernels
(moe_layout + moe_dispatch, moe_combine, moe_combine_backward,
moe_dispatch_backward); these Functions only route tensors. Use one
MoeDispatcher(backward=True) per MoE layer. The small per-call state the
backward needs (row map, true total) is copied at forward time, so a later
forward of the same layer cannot overwrite it.

The dispatched rows are another matter: by default dispatch() returns a view
of the dispatcher's persistent x_e buffer, which the layer's next forward
rewrites. An expert that saves its input for its weight gradient then sees
the newer rows. So each forward records the dispatcher's x_e generation, and
the combine's backward (which runs before the expert's backward) raises if a
later dispatch on the same dispatcher rewrote x_e in between. Schedules with
several forwards in flight per layer (pipelining with micro-batches,
activation recompute) use MoeTokenDispatcher(..., clone_x_e=True): dispatch
then returns a copy of the rows that the layer owns.
"""
from __future__ import annotations

from typing import Optional

import torch

from .moe import MoeDispatcher


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, scores, ids, disp: MoeDispatcher, ntpr: int, clone_x_e: bool):
        lay = disp.layout(ids, ntpr)
        out = disp.dispatch(x, scores.detach(), ids, lay.counts, num_tokens_per_rank=ntpr)
        row_map = lay.row_map.clone()
        total = lay.offsets[-1:].clone()
        ctx.disp, ctx.T, ctx.ntpr, ctx.row_map = disp, x.shape[0], ntpr, row_map
        ctx.mark_non_differentiable(row_map, total)
        # A fresh tensor object per call: autograd attaches this call's node to
        # it, and the binding hands out one shared view per extent.
        x_e = out.x_e.clone() if clone_x_e else out.x_e.view(out.x_e.shape)
        return x_e, row_map, total

    @staticmethod
    def backward(ctx, grad_x_e, _grad_row_map, _grad_total):
        g = grad_x_e.contiguous()
        grad_x = ctx.disp.dispatch_backward(g, ctx.row_map, ctx.T, num_tokens_per_rank=ctx.ntpr)
        return grad_x.clone(), None, None, None, None, None


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y_e, scores, row_map, total, disp: MoeDispatcher, ntpr: int,
                generation: Optional[int]):
        rows = disp.rows_for(ntpr)
        if y_e.shape[0] != rows:
            raise ValueError(f"y_e must have round_up4(num_tokens_per_rank) * topk = {rows} "
                             f"rows (the dispatched rows), got {y_e.shape[0]}")
        y = disp.combine(y_e, row_map, scores, num_tokens_per_rank=ntpr)
        ctx.save_for_backward(y_e, scores, row_map, total)
        ctx.disp, ctx.ntpr, ctx.generation = disp, ntpr, generation
        return y.clone()

    @staticmethod
    def backward(ctx, grad_y):
        if ctx.generation is not None and ctx.disp.x_e_generation != ctx.generation:
            raise RuntimeError(
                "x_e of this MoE layer was rewritten by a later dispatch before this backward "
                "(several forwards in flight on one MoeDispatcher); the expert's saved input "
                "would be the newer rows. Use MoeTokenDispatcher(..., clone_x_e=True).")
        y_e, scores, row_map, total = ctx.saved_tensors
        # The library writes the slots' rows and +0.0 into the rows from the
        # true total on (no slot reaches them), reading the total on the device.
        g_e, g_s = ctx.disp.combine_backward(grad_y.contiguous(), y_e, row_map, scores,
                                             num_tokens_per_rank=ctx.ntpr, total=total)
        return g_e.clone(), g_s.clone(), None, None, None, None, None


class MoeTokenDispatcher:
    """Differentiable dispatch/combine of one MoE layer.

        d = MoeTokenDispatcher(MoeDispatcher(nmax, D, E, K, backward=True))
        x_e = d.dispatch(x, scores, ids)        # [round_up4(ntpr) * K, D]
        y_e = experts(x_e)                      # rows [0, total) are the tokens'
        y = d.combine(y_e, scores)              # [T, D]
        y.backward(...)                         # dL/dx, dL/dscores, dL/dy_e

    clone_x_e=False (default): x_e is a view of the dispatcher's buffer and a
    second forward before the first one's backward is detected and raises.
    clone_x_e=True: x_e is a copy owned by the caller; any number of forwards
    may be in flight.
    """

    def __init__(self, dispatcher: MoeDispatcher, clone_x_e: bool = False):
        if not dispatcher.backward_enabled:
            raise ValueError("the MoeDispatcher needs backward=True")
        self.disp = dispatcher
        self.clone_x_e = bool(clone_x_e)
        self._row_map: Optional[torch.Tensor] = None
        self._total: Optional[torch.Tensor] = None
        self._ntpr: Optional[int] = None
        self._generation: Optional[int] = None

    def dispatch(self, x: torch.Tensor, topk_scores: torch.Tensor, topk_ids: torch.Tensor,
                 num_tokens_per_rank: Optional[int] = None) -> torch.Tensor:
        ntpr = x.shape[0] if num_tokens_per_rank is None else int(num_tokens_per_rank)
        x_e, self._row_map, self._total = _Dispatch.apply(
            x.contiguous(), topk_scores.contiguous(), topk_ids.contiguous(), self.disp, ntpr,
            self.clone_x_e)
        self._ntpr = ntpr
        self._generation = None if self.clone_x_e else self.disp.x_e_generation
        return x_e

    def combine(self, y_e: torch.Tensor, topk_scores: torch.Tensor) -> torch.Tensor:
        if self._row_map is None:
            raise RuntimeError("combine() needs a preceding dispatch() on this layer")
        return _Combine.apply(y_e.contiguous(), topk_scores.contiguous(), self._row_map,
                              self._total, self.disp, self._ntpr, self._generation)
