"""Pins for the backward oracle (oracle/monarch_backward.py): checks that do not
come from its hand-derived formulas.

Each pin takes an implementation ``g(q, k, v, do, grid, r_axes, tile) -> (dq, dk, dv)``
so that the same checks also run against broken copies (planted mistakes, CPU only).

Sources of truth:
* automatic differentiation: torch float64 autograd through the forward operator
  written as the explicit product of per-stage softmax matrices (built from the
  token sets with index arithmetic, independently of the oracle's loops);
* central finite differences of the forward oracle along random directions;
* the degenerate block spec r_axes = 3 (one block, stage L trivial), where the
  gradient is that of textbook dense attention: torch's CPU float64
  ``scaled_dot_product_attention`` differentiated by autograd;
* invariants: summed over all tokens, dV equals the sum of dO (both factors
  are row-stochastic); the gradient is linear in dO.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import monarch_backward as mb

GRID = (2, 4, 4)


def _oracle_bwd(q, k, v, do, grid, r_axes=1, tile=None):
    return mb.monarch_attention_backward(q, k, v, do, grid, r_axes=r_axes, tile=tile)


def _rand(grid, d=8, heads=2, seed=11, n_arrays=4):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((1, heads, n, d)) for _ in range(n_arrays)]


def _torch_forward(q, k, v, grid, r_axes, tile):
    """O = M(Q, K) V with M built from masks: M = L_perm R, where R and L are
    row softmaxes of s Q K^T restricted (by -inf) to same-stage-R-block and
    same-stage-L-set token pairs."""
    T, H, W = grid
    N = T * H * W
    d = q.shape[-1]
    n = torch.arange(N)
    b1, b2 = oracle.block_sizes(grid, r_axes)
    blk, intra = n // b2, n % b2
    same_r = blk[:, None] == blk[None, :]
    same_l = intra[:, None] == intra[None, :]
    if tile is not None:
        t, h = (n // W) // H, (n // W) % H
        box = (t // tile[0]) * 100000 + (h // tile[1])
        same_l = same_l & (box[:, None] == box[None, :])
    logits = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    ninf = torch.tensor(float("-inf"), dtype=logits.dtype)
    R = torch.softmax(torch.where(same_r, logits, ninf), dim=-1)
    L = torch.softmax(torch.where(same_l, logits, ninf), dim=-1)
    return L @ (R @ v)


def _autograd(q, k, v, do, grid, r_axes, tile):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = _torch_forward(qt, kt, vt, grid, r_axes, tile)
    (out * torch.from_numpy(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _close(a, b, tol):
    return all(np.allclose(x, y, rtol=0, atol=tol) for x, y in zip(a, b))


SPECS = [(1, None), (2, None), (0, None), (1, (1, 2)), (1, (2, 2))]


# ---------------------------------------------------------------- pins
def pin_autograd(g):
    q, k, v, do = _rand(GRID)
    return all(_close(g(q, k, v, do, GRID, r, t), _autograd(q, k, v, do, GRID, r, t), 1e-10) for r, t in SPECS)


def pin_finite_differences(g):
    q, k, v, do = _rand(GRID, seed=12)
    rng = np.random.default_rng(13)
    eps = 1e-5
    ok = True
    for r, t in [(1, None), (1, (2, 2))]:
        grads = g(q, k, v, do, GRID, r, t)
        for which in range(3):
            e = rng.standard_normal(q.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + eps * e
            args_m[which] = args_m[which] - eps * e
            fp = oracle.monarch_attention(*args_p, GRID, r_axes=r, tile=t)
            fm = oracle.monarch_attention(*args_m, GRID, r_axes=r, tile=t)
            numeric = float(((fp - fm) / (2 * eps) * do).sum())
            analytic = float((grads[which] * e).sum())
            ok &= abs(numeric - analytic) <= 1e-6 * max(1.0, abs(analytic))
    return ok


def pin_dense_reduction(g):
    q, k, v, do = _rand(GRID, seed=14)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    (out * torch.from_numpy(do)).sum().backward()
    ref = (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy())
    return _close(g(q, k, v, do, GRID, 3, None), ref, 1e-10)


def pin_dv_sum(g):
    q, k, v, do = _rand(GRID, seed=15)
    ok = True
    for r, t in SPECS:
        _, _, dv = g(q, k, v, do, GRID, r, t)
        ok &= np.allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-10)
    return ok


def pin_linear_in_dout(g):
    q, k, v, do1, do2 = _rand(GRID, seed=16, n_arrays=5)
    a, b = 0.7, -1.9
    lhs = g(q, k, v, a * do1 + b * do2, GRID, 1, None)
    g1 = g(q, k, v, do1, GRID, 1, None)
    g2 = g(q, k, v, do2, GRID, 1, None)
    return _close(lhs, [a * x + b * y for x, y in zip(g1, g2)], 1e-10)


PINS = [pin_autograd, pin_finite_differences, pin_dense_reduction, pin_dv_sum, pin_linear_in_dout]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_passes_pin(pin):
    assert pin(_oracle_bwd)


def test_backward_at_workload_shape_is_finite_and_sums():
    from workloads import WORKLOADS, make_qkv
    wl = WORKLOADS["chunk"]
    q, k, v = make_qkv(wl, heads=1)
    do = np.random.default_rng(3).standard_normal(q.shape)
    dq, dk, dv = _oracle_bwd(q, k, v, do, (wl.T, wl.H, wl.W))
    assert all(np.isfinite(x).all() for x in (dq, dk, dv))
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-9)


# ---------------------------------------------------------------- planted mistakes
def _mut_no_rowsum(q, k, v, do, grid, r_axes=1, tile=None):
    # dS = P * dP (drops the - D term)
    orig = mb.group_softmax_attention_backward

    def broken(qq, kk, vv, dd, groups):
        s = 1.0 / math.sqrt(qq.shape[-1])
        dq, dk, dv = np.zeros_like(qq), np.zeros_like(kk), np.zeros_like(vv)
        for gset in groups:
            lg = s * (qq[gset] @ kk[gset].T)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dv[gset] = p.T @ dd[gset]
            dsc = p * (dd[gset] @ vv[gset].T)
            dq[gset] = s * dsc @ kk[gset]
            dk[gset] = s * dsc.T @ qq[gset]
        return dq, dk, dv
    mb.group_softmax_attention_backward = broken
    try:
        return mb.monarch_attention_backward(q, k, v, do, grid, r_axes, tile)
    finally:
        mb.group_softmax_attention_backward = orig


def _mut_dk_not_transposed(q, k, v, do, grid, r_axes=1, tile=None):
    dq, dk, dv = mb.monarch_attention_backward(k, q, v, do, grid, r_axes, tile)   # roles of q and k swapped
    return dk, dq, dv


def _mut_drop_stage_l_terms(q, k, v, do, grid, r_axes=1, tile=None):
    dq, dk, dv, parts = mb.monarch_attention_backward(q, k, v, do, grid, r_axes, tile, return_parts=True)
    return parts["dq_r"], parts["dk_r"], dv


def _mut_dv_from_do(q, k, v, do, grid, r_axes=1, tile=None):
    # stage R fed dO instead of dY (skips the chain through stage L)
    dq_l, dk_l, _ = mb.stage_l_backward(q, k, oracle.stage_r(q, k, v, grid, r_axes), do, grid, r_axes, tile)
    dq_r, dk_r, dv = mb.stage_r_backward(q, k, v, do, grid, r_axes)
    return dq_l + dq_r, dk_l + dk_r, dv


def _mut_missing_scale(q, k, v, do, grid, r_axes=1, tile=None):
    dq, dk, dv = mb.monarch_attention_backward(q, k, v, do, grid, r_axes, tile)
    d = np.asarray(q).shape[-1]
    return dq * math.sqrt(d), dk * math.sqrt(d), dv


def _mut_tile_ignored(q, k, v, do, grid, r_axes=1, tile=None):
    return mb.monarch_attention_backward(q, k, v, do, grid, r_axes, None)


MUTANTS = [_mut_no_rowsum, _mut_dk_not_transposed, _mut_drop_stage_l_terms, _mut_dv_from_do,
           _mut_missing_scale, _mut_tile_ignored]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_backward_mistake_fails_a_pin(mutant):
    failed = []
    for pin in PINS:
        try:
            ok = pin(mutant)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, "no pin catches %s" % mutant.__name__
