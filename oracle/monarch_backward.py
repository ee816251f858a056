"""Backward pass of Monarch attention -- CPU oracle, TEST INFRASTRUCTURE ONLY.

Only the tests may import this module. The HIP library never calls it and
shares no code with it.

The pages say the method's custom kernels run both the forward and the
backward pass, tiled like FlashAttention so that no dense attention matrix is
materialised [it, "Finetuning e Implementazione Efficiente"; pt, 2; fr, 2.C;
nl, "Finetuning en Geoptimaliseerde Implementatie"; zh, 微调与高效实现]. They
print no backward equations. The gradient of the forward operator of
``monarch.py`` is fixed by the chain rule, and this module writes it out.

For one token set G of one stage (s = 1/sqrt(d)):

    forward:   S = s Q_G K_G^T,   P = softmax_rows(S),   O_G = P V_G
    backward:  dV_G = P^T dO_G
               dP   = dO_G V_G^T
               dS   = P * (dP - D),   D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
               dQ_G = s dS K_G,       dK_G = s dS^T Q_G

The two stages compose as O = stage_L(Q, K, Y) with Y = stage_R(Q, K, V):
stage L's backward gives (dQ_L, dK_L, dY); stage R's backward, fed dY, gives
(dQ_R, dK_R, dV); then dQ = dQ_L + dQ_R and dK = dK_L + dK_R. Float64 NumPy
throughout; loops over token sets as in the forward oracle.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from .monarch import stage_l_groups, stage_r_groups, group_softmax_attention

__all__ = [
    "group_softmax_attention_backward",
    "stage_r_backward",
    "stage_l_backward",
    "monarch_attention_backward",
]


def group_softmax_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                                     groups: Sequence[np.ndarray]):
    """(dq, dk, dv) of out[G] = softmax_rows(s q[G] k[G]^T) v[G] for every set G, given dout.

    q, k, v, do: [N, d] float64 for one (batch, head); the sets partition the tokens.
    """
    d = q.shape[-1]
    s = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for g in groups:
        logits = s * (q[g] @ k[g].T)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dv[g] = p.T @ do[g]
        dp = do[g] @ v[g].T
        dsc = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[g] = s * (dsc @ k[g])
        dk[g] = s * (dsc.T @ q[g])
    return dq, dk, dv


def _per_head3(fn, *arrays):
    arrays = [np.asarray(a, dtype=np.float64) for a in arrays]
    B, Hh = arrays[0].shape[:2]
    outs = [np.empty(arrays[0].shape, dtype=np.float64) for _ in range(3)]
    for b in range(B):
        for h in range(Hh):
            res = fn(*[a[b, h] for a in arrays])
            for o, r in zip(outs, res):
                o[b, h] = r
    return tuple(outs)


def stage_r_backward(q, k, v, dy, grid, r_axes: int = 1):
    """(dq_R, dk_R, dv) of Y = stage_R(Q, K, V) given dY."""
    groups = stage_r_groups(grid, r_axes)
    return _per_head3(lambda qq, kk, vv, gg: group_softmax_attention_backward(qq, kk, vv, gg, groups),
                      q, k, v, dy)


def stage_l_backward(q, k, y, do, grid, r_axes: int = 1, tile=None):
    """(dq_L, dk_L, dy) of O = stage_L(Q, K, Y) given dO."""
    groups = stage_l_groups(grid, r_axes, tile)
    return _per_head3(lambda qq, kk, yy, gg: group_softmax_attention_backward(qq, kk, yy, gg, groups),
                      q, k, y, do)


def monarch_attention_backward(q, k, v, do, grid: Tuple[int, int, int], r_axes: int = 1, tile=None,
                               return_parts: bool = False):
    """(dq, dk, dv) of O = P L P^T R V (the forward of monarch.py) given dO; float64.

    With return_parts, also returns a dict with the per-stage terms and dY.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    r_groups = stage_r_groups(grid, r_axes)
    y = np.empty_like(v)
    B, Hh = q.shape[:2]
    for b in range(B):
        for h in range(Hh):
            y[b, h] = group_softmax_attention(q[b, h], k[b, h], v[b, h], r_groups)
    dq_l, dk_l, dy = stage_l_backward(q, k, y, do, grid, r_axes, tile)
    dq_r, dk_r, dv = stage_r_backward(q, k, v, dy, grid, r_axes)
    dq, dk = dq_l + dq_r, dk_l + dk_r
    if return_parts:
        return dq, dk, dv, {"dq_l": dq_l, "dk_l": dk_l, "dy": dy, "dq_r": dq_r, "dk_r": dk_r, "y": y}
    return dq, dk, dv

