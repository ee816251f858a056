"""torch.autograd wrapper of the bf16 Monarch attention entry points.

``monarch_attention(q, k, v, T, H, W, r_axes=1, tile=None)`` runs
``monarch_attn_fwd`` (or ``monarch_attn_tiled_fwd`` when ``tile`` is given)
and, when gradients are needed, keeps the forward's workspace (stage R's output
Y) for ``monarch_attn_bwd``, which then skips recomputing stage R. Allocation
of outputs and workspaces and the choice of entry point are all that happens
here; both passes run in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _binding as B


def _workspace(q: torch.Tensor, nbytes: int) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 1) // 2, dtype=torch.bfloat16, device=q.device)


class MonarchAttention(torch.autograd.Function):
    """Monarch-factored attention over a (T, H, W) token grid; tensors
    [batch, heads, T*H*W, head_dim], bf16, contiguous, on the GPU."""

    @staticmethod
    def forward(ctx, q, k, v, T, H, W, r_axes=1, tile=None):
        if q.dtype != torch.bfloat16:
            raise TypeError("monarch_attention takes bf16 tensors (the backward is bf16 only)")
        q, k, v = (x.contiguous() for x in (q, k, v))
        B_, h, N, d = q.shape
        tt, th = tile if tile is not None else (0, 0)
        r = 1 if tile is not None else r_axes
        ws = _workspace(q, B.ma_workspace_bytes(B_, h, T, H, W, r, tt, th, d, B.MA_BF16))
        out = torch.empty_like(q)
        if tile is not None:
            B.monarch_attn_tiled_fwd(q, k, v, out, ws, T, H, W, tt, th)
        else:
            B.monarch_attn_fwd(q, k, v, out, ws, T, H, W, r_axes)
        ctx.grid = (T, H, W, r, tt, th)
        ctx.save_for_backward(q, k, v, out, ws if ws is not None else torch.empty(0, device=q.device))
        ctx.has_y = ws is not None
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, ws = ctx.saved_tensors
        T, H, W, r, tt, th = ctx.grid
        dout = dout.contiguous().to(torch.bfloat16)
        B_, h, N, d = q.shape
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        wsb = _workspace(q, B.ma_bwd_workspace_bytes(B_, h, T, H, W, r, tt, th, d, B.MA_BF16))
        y = ws[:q.numel()].view(q.shape) if ctx.has_y else None
        B.monarch_attn_bwd(q, k, v, out, dout, dq, dk, dv, wsb, T, H, W, r, tt, th, y=y)
        return dq, dk, dv, None, None, None, None, None


def monarch_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, T: int, H: int, W: int,
                      r_axes: int = 1, tile: Optional[Tuple[int, int]] = None) -> torch.Tensor:
    """Monarch attention of (q, k, v) with autograd support (bf16)."""
    return MonarchAttention.apply(q, k, v, T, H, W, r_axes, tile)
