"""CPU oracle for Monarch-factored video attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this module. The HIP library never calls it and shares no code with it.

Plain, slow, float64 NumPy. Every function follows a definition that can be
checked by eye:

* Source pages: the gist.science summaries of arXiv 2602.12271, "MonarchRT:
  Efficient Attention for Real-Time Video Generation" (it / pt / fr / nl / zh).
  Cited below as e.g. ``[nl, Methodologie]`` or ``[zh, 2.2]``.
* The attention matrix is factored as a product of permutation and
  block-diagonal matrices [nl, Methodologie]; P is a permutation [zh, 2.1].
* Block sizes are aligned with the video axes, e.g. (b1, b2) = (f*h, w), with
  b1*b2 = N [zh, 2.2 block alignment; pt, 2.B]. Here the trailing ``r_axes``
  grid axes form one block of length b2 and b1 = N / b2.
* Reading used for the factors (the pages print no equations for them): the
  right factor blockdiag(R_0..R_{b1-1}) holds, per block of b2 contiguous
  tokens, the row softmax of s*Q K^T restricted to that block ("stage R"); the
  left factor P blockdiag(L_0..L_{b2-1}) P^T holds, per intra-block index i,
  the row softmax of s*Q K^T over the b1 tokens {a*b2 + i} ("stage L"). Both use
  the original Q and K, s = 1/sqrt(head_dim), and M = P L P^T R acts on V with R
  first: O = M V.
* Tiled Monarch [zh, 2.2 tiled Monarch; fr, 2.B; nl, Methodologie]: each stage-L
  group is split into (tile_t frames x tile_h rows) boxes at a fixed w, and the
  softmax of stage L runs inside a box only. The last box along an axis may be
  shorter when the axis length is not a multiple of the tile.
* Dense attention softmax(s*Q K^T) V over all N tokens is the quadratic-cost
  operator the method replaces [it, 1; zh, overview].

Arrays are ``[batch, heads, N, d]`` with token ``n = (t*H + h)*W + w``.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "block_sizes",
    "stage_r_groups",
    "stage_l_groups",
    "group_softmax_attention",
    "stage_r",
    "stage_l",
    "monarch_attention",
    "monarch_attention_rows",
    "dense_attention",
    "dense_attention_rows",
    "explicit_monarch_matrix",
]


def block_sizes(grid: Tuple[int, int, int], r_axes: int = 1) -> Tuple[int, int]:
    """(b1, b2) for a (T, H, W) grid whose trailing ``r_axes`` axes form a block.

    r_axes = 1: b2 = W, b1 = T*H   (the (f*h, w) split of [zh, 2.2])
    r_axes = 2: b2 = H*W, b1 = T   (the (f, h*w) split)
    r_axes = 3: b2 = N, b1 = 1     (one block: stage L is trivial)
    r_axes = 0: b2 = 1, b1 = N     (stage R is trivial)
    """
    T, H, W = grid
    if r_axes == 0:
        b2 = 1
    elif r_axes == 1:
        b2 = W
    elif r_axes == 2:
        b2 = H * W
    elif r_axes == 3:
        b2 = T * H * W
    else:
        raise ValueError("r_axes must be 0..3")
    return (T * H * W) // b2, b2


def stage_r_groups(grid, r_axes: int = 1) -> List[np.ndarray]:
    """Blocks of b2 contiguous tokens: block a = {a*b2 + j : j < b2}."""
    b1, b2 = block_sizes(grid, r_axes)
    return [np.arange(a * b2, (a + 1) * b2) for a in range(b1)]


def stage_l_groups(grid, r_axes: int = 1, tile: Optional[Tuple[int, int]] = None) -> List[np.ndarray]:
    """Token sets of stage L.

    Untiled: for each intra-block index i, {a*b2 + i : a < b1} (stride b2).
    Tiled (needs r_axes = 1, so a = t*H + h): for each w and each box
    {(t, h): t // tile_t = tt, h // tile_h = th}, the tokens (t*H + h)*W + w.
    """
    T, H, W = grid
    b1, b2 = block_sizes(grid, r_axes)
    if tile is None:
        return [np.arange(i, b1 * b2, b2) for i in range(b2)]
    if r_axes != 1:
        raise ValueError("tiles are defined on the (frame, row) axes of stage L: r_axes must be 1")
    tile_t, tile_h = tile
    if tile_t < 1 or tile_h < 1:
        raise ValueError("tile sizes must be >= 1")
    groups = []
    for w in range(W):
        for t0 in range(0, T, tile_t):
            for h0 in range(0, H, tile_h):
                members = []
                for t in range(t0, min(T, t0 + tile_t)):
                    for h in range(h0, min(H, h0 + tile_h)):
                        members.append((t * H + h) * W + w)
                groups.append(np.array(members, dtype=np.int64))
    return groups


def group_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                            groups: Sequence[np.ndarray]) -> np.ndarray:
    """For each token set G: out[G] = softmax_rows(s * q[G] k[G]^T) v[G].

    q, k, v: [N, d] float64 for one (batch, head). The sets must partition
    the tokens. Softmax is max-subtracted for range only; it does not change
    the value.
    """
    d = q.shape[-1]
    s = 1.0 / math.sqrt(d)
    out = np.full(v.shape, np.nan, dtype=np.float64)
    for g in groups:
        logits = s * (q[g] @ k[g].T)
        logits = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[g] = p @ v[g]
    return out


def _per_head(fn, *arrays):
    arrays = [np.asarray(a, dtype=np.float64) for a in arrays]
    B, Hh = arrays[0].shape[:2]
    out = np.empty(arrays[-1].shape, dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            out[b, h] = fn(*[a[b, h] for a in arrays])
    return out


def stage_r(q, k, v, grid, r_axes: int = 1) -> np.ndarray:
    """Y = blockdiag(R) V: per block of b2 contiguous tokens, softmax attention."""
    groups = stage_r_groups(grid, r_axes)
    return _per_head(lambda qq, kk, vv: group_softmax_attention(qq, kk, vv, groups), q, k, v)


def stage_l(q, k, y, grid, r_axes: int = 1, tile=None) -> np.ndarray:
    """O = P blockdiag(L) P^T Y: softmax attention over each stage-L token set."""
    groups = stage_l_groups(grid, r_axes, tile)
    return _per_head(lambda qq, kk, yy: group_softmax_attention(qq, kk, yy, groups), q, k, y)


def monarch_attention(q, k, v, grid, r_axes: int = 1, tile=None, return_y: bool = False):
    """O = P L P^T R V for q, k, v of shape [batch, heads, T*H*W, d] (float64 result)."""
    T, H, W = grid
    if np.asarray(q).shape[-2] != T * H * W:
        raise ValueError("token count does not match the grid")
    y = stage_r(q, k, v, grid, r_axes)
    o = stage_l(q, k, y, grid, r_axes, tile)
    return (o, y) if return_y else o


def _softmax_row(logits: np.ndarray) -> np.ndarray:
    p = np.exp(logits - logits.max())
    return p / p.sum()


def monarch_attention_rows(q, k, v, grid, rows: Sequence[int], r_axes: int = 1,
                           tile=None) -> np.ndarray:
    """The same operator evaluated only at token indices ``rows``.

    Returns [batch, heads, len(rows), d]. For an output token n in stage-L set
    G_L(n): o_n = sum_{m in G_L(n)} softmax_m(s q_n.k_m) y_m, where each
    y_m = sum_{j in block(m)} softmax_j(s q_m.k_j) v_j is evaluated directly.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hh, N, d = q.shape
    s = 1.0 / math.sqrt(d)
    b1, b2 = block_sizes(grid, r_axes)
    l_groups = stage_l_groups(grid, r_axes, tile)
    owner = np.empty(N, dtype=np.int64)
    for gi, g in enumerate(l_groups):
        owner[g] = gi
    out = np.empty((B, Hh, len(rows), d), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            qq, kk, vv = q[b, h], k[b, h], v[b, h]
            for r, n in enumerate(rows):
                members = l_groups[owner[n]]
                ys = np.empty((members.size, d))
                for mi, m in enumerate(members):
                    blk = np.arange((m // b2) * b2, (m // b2 + 1) * b2)
                    ys[mi] = _softmax_row(s * (kk[blk] @ qq[m])) @ vv[blk]
                out[b, h, r] = _softmax_row(s * (kk[members] @ qq[n])) @ ys
    return out


def dense_attention(q, k, v) -> np.ndarray:
    """softmax(s Q K^T) V over all tokens, per (batch, head)."""
    def one(qq, kk, vv):
        return group_softmax_attention(qq, kk, vv, [np.arange(qq.shape[0])])
    return _per_head(one, q, k, v)


def dense_attention_rows(q, k, v, rows: Sequence[int]) -> np.ndarray:
    """Dense attention evaluated only at query tokens ``rows``: [batch, heads, len(rows), d]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hh, N, d = q.shape
    s = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((B, Hh, rows.size, d))
    for b in range(B):
        for h in range(Hh):
            logits = s * (q[b, h, rows] @ k[b, h].T)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = p @ v[b, h]
    return out


def explicit_monarch_matrix(q, k, grid, r_axes: int = 1, tile=None) -> np.ndarray:
    """Brute force for tiny grids: build M = P . blockdiag(L) . P^T . blockdiag(R).

    q, k: [N, d] for one head. Every factor is written out as an N x N matrix
    with explicit loops:
      R[a*b2+i, a*b2+j]  = exp(s q_{a*b2+i}.k_{a*b2+j}) / sum_j' (same, j')
      Lp[i*b1+a, i*b1+c] = exp(s q_{a*b2+i}.k_{c*b2+i}) / sum over c' in the
                           stage-L set of a (all of [b1], or a's tile box)
      P[a*b2+i, i*b1+a]  = 1   (so (P^T x)[i*b1+a] = x[a*b2+i])
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N, d = q.shape
    s = 1.0 / math.sqrt(d)
    T, H, W = grid
    b1, b2 = block_sizes(grid, r_axes)
    if tile is not None and r_axes != 1:
        raise ValueError("tiles need r_axes = 1")
    R = np.zeros((N, N))
    for a in range(b1):
        for i in range(b2):
            row = [math.exp(s * float(np.dot(q[a * b2 + i], k[a * b2 + j]))) for j in range(b2)]
            tot = sum(row)
            for j in range(b2):
                R[a * b2 + i, a * b2 + j] = row[j] / tot

    def same_set(a: int, c: int) -> bool:
        if tile is None:
            return True
        t_a, h_a = divmod(a, H)
        t_c, h_c = divmod(c, H)
        return t_a // tile[0] == t_c // tile[0] and h_a // tile[1] == h_c // tile[1]

    Lp = np.zeros((N, N))
    for i in range(b2):
        for a in range(b1):
            cols = [c for c in range(b1) if same_set(a, c)]
            row = {c: math.exp(s * float(np.dot(q[a * b2 + i], k[c * b2 + i]))) for c in cols}
            tot = sum(row.values())
            for c in cols:
                Lp[i * b1 + a, i * b1 + c] = row[c] / tot
    P = np.zeros((N, N))
    for a in range(b1):
        for i in range(b2):
            P[a * b2 + i, i * b1 + a] = 1.0
    return P @ Lp @ P.T @ R
