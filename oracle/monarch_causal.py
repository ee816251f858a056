"""Chunk-causal Monarch attention -- CPU oracle, TEST INFRASTRUCTURE ONLY.

Only the tests may import this module. The HIP library never calls it and
shares no code with it.

The pages' real-time target is autoregressive, chunk-by-chunk video
generation, where errors accumulate over time and every denoising step has to
process a lot of information [it, 1; fr, 1; zh, 1]; the autoregressive model
they evaluate (Self-Forcing) generates a few frames at a time [it, 3; fr, 4].
They never define Monarch attention over such a causal sequence. Reading used
here:

* Frames are split into chunks of ``chunk_t`` consecutive frames, chunk(t) =
  t div chunk_t. A token may use the keys of its own chunk and of earlier
  chunks only (block-causal at chunk granularity, bidirectional inside a
  chunk).
* Stage R is unchanged: its blocks are W-rows (r_axes = 1), whole frames
  (r_axes = 2) or single tokens (r_axes = 0), so no block crosses a frame and
  stage R is causal as it stands. r_axes = 3 (one block over every frame) is
  not causal and is rejected.
* Stage L for a query token keeps its group (the tokens at the same intra-block
  index) but restricts the softmax to members whose frame lies in the query's
  chunk or an earlier one. Values are Y, as in the bidirectional operator.
* One autoregressive step with a cache: the chunk of frames [t0, t0 + chunk_t)
  computes its Y (stage R inside its own frames) and its O from stage L over
  the members in frames [0, t0 + chunk_t), whose Y for frames before t0 comes
  from the cache.

Float64 NumPy; per stage-L group and per chunk the softmax is one matrix
product over the allowed keys.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

from .monarch import group_softmax_attention, stage_l_groups, stage_r, stage_r_groups

__all__ = [
    "member_frames",
    "causal_stage_l",
    "monarch_attention_causal",
    "monarch_attention_chunk_step",
]


def _check(grid, r_axes, chunk_t):
    if r_axes not in (0, 1, 2):
        raise ValueError("chunk-causal Monarch needs stage-R blocks inside one frame: r_axes in 0..2")
    if chunk_t < 1:
        raise ValueError("chunk_t must be >= 1")


def member_frames(grid: Tuple[int, int, int]) -> np.ndarray:
    """Frame of every token, indexed by token: t = n div (H*W)."""
    T, H, W = grid
    return np.arange(T * H * W, dtype=np.int64) // (H * W)


def causal_stage_l(q, k, y, grid, chunk_t: int, r_axes: int = 1) -> np.ndarray:
    """O[n] = softmax over {m in G_L(n) : chunk(frame m) <= chunk(frame n)} of s q_n.k_m, applied to y."""
    _check(grid, r_axes, chunk_t)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    y = np.asarray(y, np.float64)
    B, Hh, N, d = q.shape
    s = 1.0 / math.sqrt(d)
    chunk_of = member_frames(grid) // chunk_t
    out = np.full(y.shape, np.nan)
    for g in stage_l_groups(grid, r_axes):
        cg = chunk_of[g]
        for c in np.unique(cg):
            rows = g[cg == c]
            keys = g[cg <= c]
            for b in range(B):
                for h in range(Hh):
                    logits = s * (q[b, h, rows] @ k[b, h, keys].T)
                    logits -= logits.max(axis=1, keepdims=True)
                    p = np.exp(logits)
                    p /= p.sum(axis=1, keepdims=True)
                    out[b, h, rows] = p @ y[b, h, keys]
    return out


def monarch_attention_causal(q, k, v, grid, chunk_t: int, r_axes: int = 1, return_y: bool = False):
    """Chunk-causal Monarch over the whole sequence: stage R as usual, then causal stage L."""
    _check(grid, r_axes, chunk_t)
    T, H, W = grid
    if np.asarray(q).shape[-2] != T * H * W:
        raise ValueError("token count does not match the grid")
    y = stage_r(q, k, v, grid, r_axes)
    o = causal_stage_l(q, k, y, grid, chunk_t, r_axes)
    return (o, y) if return_y else o


def monarch_attention_chunk_step(q, k, v, y_cache, grid, t0: int, chunk_t: int, r_axes: int = 1):
    """One step with a cache: returns (y_chunk, o_chunk), each [B, heads, chunk tokens, d].

    q, k, v, y_cache are whole-grid arrays [B, heads, T*H*W, d]; only frames
    [0, t0 + chunk_t) are read, and y_cache only for frames [0, t0). The chunk's
    Y is stage R over its own blocks; its O is stage L over the members of each
    group that lie in frames [0, t0 + chunk_t), with values from y_cache before
    t0 and from the new Y inside the chunk.
    """
    _check(grid, r_axes, chunk_t)
    T, H, W = grid
    if t0 < 0 or t0 + chunk_t > T:
        raise ValueError("the chunk must lie inside the grid")
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hh, N, d = q.shape
    fsz = H * W
    lo, hi = t0 * fsz, (t0 + chunk_t) * fsz
    # stage R over the blocks of the chunk's frames (each block lies in one frame)
    y = np.array(y_cache, dtype=np.float64, copy=True)
    y[:, :, hi:] = np.nan   # frames after the chunk are not part of this step
    chunk_blocks = [blk for blk in stage_r_groups(grid, r_axes) if lo <= blk[0] and blk[-1] < hi]
    for b in range(B):
        for h in range(Hh):
            full = group_softmax_attention(q[b, h], k[b, h], v[b, h], chunk_blocks)
            y[b, h, lo:hi] = full[lo:hi]
    # stage L: every group's members in frames [0, t0 + chunk_t); queries in the chunk
    s = 1.0 / math.sqrt(d)
    o = np.full((B, Hh, hi - lo, d), np.nan)
    for g in stage_l_groups(grid, r_axes):
        keys = g[g < hi]
        rows = g[(g >= lo) & (g < hi)]
        for b in range(B):
            for h in range(Hh):
                logits = s * (q[b, h, rows] @ k[b, h, keys].T)
                logits -= logits.max(axis=1, keepdims=True)
                p = np.exp(logits)
                p /= p.sum(axis=1, keepdims=True)
                o[b, h, rows - lo] = p @ y[b, h, keys]
    return y[:, :, lo:hi], o
