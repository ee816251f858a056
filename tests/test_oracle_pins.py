"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each pin takes an implementation ``f(q, k, v, grid, r_axes, tile) -> O`` so that
the same checks also run against deliberately broken copies of the oracle
(planted mistakes, CPU only) to show that a plausible error fails at least one.

Sources of truth used here:
* hand-derived closed forms on tiny grids (tests/golden/hand_cases.json);
* textbook dense attention computed by torch's CPU float64
  ``scaled_dot_product_attention`` in the two degenerate block specs, where
  the factored operator has one non-trivial stage spanning all tokens;
* invariants of a product of row-stochastic factors: V = 1 gives 1, linearity in V,
  Q = 0 gives block/box means, commuting with grid permutations that respect
  the block spec;
* the hard-attention limit, where each factor becomes a one-hot selection whose
  route is found by two argmaxes;
* the explicit N x N factor matrices built with loops.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
TINY = WORKLOADS["tiny"]
GRID = (TINY.T, TINY.H, TINY.W)


def _oracle_impl(q, k, v, grid, r_axes=1, tile=None):
    return oracle.monarch_attention(q, k, v, grid, r_axes=r_axes, tile=tile)


def _rand(grid, d=16, heads=2, seed=5):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((1, heads, n, d)) for _ in range(3)]


def _sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(q, np.float64)),
        torch.from_numpy(np.asarray(k, np.float64)),
        torch.from_numpy(np.asarray(v, np.float64))).numpy()


# ---------------------------------------------------------------- pins
def pin_hand_golden(f):
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    ok = True
    for c in cases:
        grid = tuple(c["grid"])
        n = grid[0] * grid[1] * grid[2]
        kv = []
        for s in c["k"]:
            s = s.strip()
            kv.append(0.0 if s == "0" else math.log(float(s.split()[-1])))
        q = np.array(c["q"], np.float64).reshape(1, 1, n, 1)
        k = np.array(kv, np.float64).reshape(1, 1, n, 1)
        v = np.array(c["v"], np.float64).reshape(1, 1, n, 1)
        tile = tuple(c["tile"]) if c["tile"] else None
        o = f(q, k, v, grid, c["r_axes"], tile)
        ok &= np.allclose(o.reshape(-1), c["o"], rtol=0, atol=1e-12)
    return ok


def pin_degenerate_dense(f):
    q, k, v = _rand(GRID)
    ref = _sdpa(q, k, v)
    a = f(q, k, v, GRID, 3, None)     # one block of N tokens: stage L trivial
    b = f(q, k, v, GRID, 0, None)     # blocks of one token: stage R trivial
    return np.allclose(a, ref, atol=1e-12) and np.allclose(b, ref, atol=1e-12)


def pin_row_stochastic(f):
    q, k, _ = _rand(GRID)
    ok = True
    for tile in (None, (1, 2), (2, 3)):
        ones = np.ones_like(q)
        ok &= np.allclose(f(q, k, ones, GRID, 1, tile), 1.0, atol=1e-12)
        ok &= np.allclose(f(q, k, -2.5 * ones, GRID, 1, tile), -2.5, atol=1e-12)
    return ok


def pin_q_zero(f):
    grid = (3, 4, 5)
    _, k, v = _rand(grid, seed=7)
    q = np.zeros_like(k)
    ok = True
    o = f(q, k, v, grid, 1, None)
    ok &= np.allclose(o, v.mean(axis=2, keepdims=True), atol=1e-12)
    tile = (2, 3)                         # ragged boxes on both axes
    o = f(q, k, v, grid, 1, tile)
    T, H, W = grid
    vg = v.reshape(1, 2, T, H, W, -1)
    exp = np.empty_like(vg)
    for t0 in range(0, T, tile[0]):
        for h0 in range(0, H, tile[1]):
            box = vg[:, :, t0:t0 + tile[0], h0:h0 + tile[1]]
            exp[:, :, t0:t0 + tile[0], h0:h0 + tile[1]] = box.mean(axis=(2, 3, 4), keepdims=True)
    ok &= np.allclose(o, exp.reshape(o.shape), atol=1e-12)
    return ok


def _permute(x, grid, perm_fn):
    T, H, W = grid
    xg = x.reshape(x.shape[0], x.shape[1], T, H, W, x.shape[-1])
    xg = perm_fn(xg)
    return np.ascontiguousarray(xg).reshape(x.shape[0], x.shape[1], -1, x.shape[-1])


def pin_permutation(f):
    ok = True
    grid = (2, 4, 4)
    q, k, v = _rand(grid, seed=9)
    flips = [lambda x: x[:, :, :, :, ::-1], lambda x: x[:, :, ::-1], lambda x: x[:, :, :, ::-1]]
    for tile in (None, (1, 2)):
        base = f(q, k, v, grid, 1, tile)
        for fl in flips:
            got = f(*[_permute(x, grid, fl) for x in (q, k, v)], grid, 1, tile)
            ok &= np.allclose(got, _permute(base, grid, fl), atol=1e-12)
    # swap the frame and row axes on a square (T = H) grid; tiles swap with them
    grid = (3, 3, 4)
    q, k, v = _rand(grid, seed=10)
    sw = lambda x: x.transpose(0, 1, 3, 2, 4, 5)
    for tile, tile_sw in ((None, None), ((1, 3), (3, 1)), ((2, 1), (1, 2))):
        base = f(q, k, v, grid, 1, tile)
        got = f(*[_permute(x, grid, sw) for x in (q, k, v)], grid, 1, tile_sw)
        ok &= np.allclose(got, _permute(base, grid, sw), atol=1e-12)
    return ok


def pin_tile_limits(f):
    q, k, v = _rand(GRID, seed=11)
    T, H, W = GRID
    ok = np.allclose(f(q, k, v, GRID, 1, (T, H)), f(q, k, v, GRID, 1, None), atol=1e-13)
    ok &= np.allclose(f(q, k, v, GRID, 1, (T + 3, H + 5)), f(q, k, v, GRID, 1, None), atol=1e-13)
    # 1x1 tiles: stage L sees one token, so O = Y = per-W-row dense attention
    o = f(q, k, v, GRID, 1, (1, 1))
    n = T * H * W
    blocks = lambda x: x.reshape(1, 2, T * H, W, -1).transpose(0, 2, 1, 3, 4).reshape(T * H * 2, 1, W, -1)
    ref = _sdpa(blocks(q), blocks(k), blocks(v)).reshape(1, T * H, 2, W, -1).transpose(0, 2, 1, 3, 4)
    ok &= np.allclose(o, ref.reshape(1, 2, n, -1), atol=1e-12)
    return ok


def pin_linearity(f):
    q, k, v1 = _rand(GRID, seed=12)
    _, _, v2 = _rand(GRID, seed=13)
    ok = True
    for tile in (None, (2, 2)):
        lhs = f(q, k, 1.5 * v1 - 0.25 * v2, GRID, 1, tile)
        rhs = 1.5 * f(q, k, v1, GRID, 1, tile) - 0.25 * f(q, k, v2, GRID, 1, tile)
        ok &= np.allclose(lhs, rhs, atol=1e-12)
    return ok


def _hard_route(q, k, grid, tile):
    """Token each output copies in the hard-attention limit (one head)."""
    T, H, W = grid
    b2 = W
    n_tok = T * H * W
    route = np.empty(n_tok, np.int64)
    for n in range(n_tok):
        a, i = divmod(n, b2)
        t, h = divmod(a, H)
        cands = []
        for a2 in range(T * H):
            t2, h2 = divmod(a2, H)
            if tile is None or (t2 // tile[0] == t // tile[0] and h2 // tile[1] == h // tile[1]):
                cands.append(a2)
        a_star = max(cands, key=lambda c: float(q[n] @ k[c * b2 + i]))
        m = a_star * b2 + i
        j_star = max(range(b2), key=lambda j: float(q[m] @ k[a_star * b2 + j]))
        route[n] = a_star * b2 + j_star
    return route


def pin_hard_route(f):
    ok = True
    for tile in (None, (1, 2)):
        q, k, v = _rand(GRID, heads=1, seed=14)
        qs = q * 1e6
        o = f(qs, k, v, GRID, 1, tile)
        route = _hard_route(q[0, 0], k[0, 0], GRID, tile)
        ok &= np.allclose(o[0, 0], v[0, 0][route], atol=1e-6)
    return ok


def pin_brute_force(f):
    q, k, v = _rand(GRID, heads=1, seed=15)
    ok = True
    for r_axes, tile in ((1, None), (1, (1, 2)), (1, (2, 3)), (2, None), (0, None), (3, None)):
        M = oracle.explicit_monarch_matrix(q[0, 0], k[0, 0], GRID, r_axes, tile)
        ok &= np.allclose(f(q, k, v, GRID, r_axes, tile)[0, 0], M @ v[0, 0], atol=1e-12)
    return ok


PINS = [pin_hand_golden, pin_degenerate_dense, pin_row_stochastic, pin_q_zero, pin_permutation,
        pin_tile_limits, pin_linearity, pin_hard_route, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(_oracle_impl)


# ---------------------------------------------------------------- structural facts of M
def test_explicit_matrix_structure():
    """M >= 0, rows sum to 1, and the (a,j) slice at fixed (i,a') is rank one."""
    q, k, _ = _rand(GRID, heads=1, seed=16)
    M = oracle.explicit_monarch_matrix(q[0, 0], k[0, 0], GRID, 1, None)
    assert (M >= 0).all()
    assert np.allclose(M.sum(axis=1), 1.0, atol=1e-13)
    T, H, W = GRID
    b1, b2 = T * H, W
    M4 = M.reshape(b1, b2, b1, b2)           # [a, i, a', j]
    for i in range(b2):
        for a2 in range(b1):
            sv = np.linalg.svd(M4[:, i, a2, :], compute_uv=False)
            assert sv[1] <= 1e-12 * max(sv[0], 1e-300)
    assert (M > 0).all()                       # two hops reach every key: dense


def test_rows_variant_matches_full():
    for name, tile in (("tiny", None), ("tiny", (1, 2)), ("tiny", (2, 3))):
        wl = WORKLOADS[name]
        q, k, v = make_qkv(wl)
        grid = (wl.T, wl.H, wl.W)
        full = oracle.monarch_attention(q, k, v, grid, tile=tile)
        rows = [0, 5, 17, 31]
        got = oracle.monarch_attention_rows(q, k, v, grid, rows, tile=tile)
        assert np.allclose(got, full[:, :, rows], atol=1e-13)
    q, k, v = _rand((2, 3, 5), d=8, seed=17)
    full = oracle.monarch_attention(q, k, v, (2, 3, 5), r_axes=2)
    got = oracle.monarch_attention_rows(q, k, v, (2, 3, 5), [1, 29], r_axes=2)
    assert np.allclose(got, full[:, :, [1, 29]], atol=1e-13)


def test_dense_matches_library():
    q, k, v = _rand((2, 3, 7), d=16, seed=18)
    ref = _sdpa(q, k, v)
    assert np.allclose(oracle.dense_attention(q, k, v), ref, atol=1e-12)
    assert np.allclose(oracle.dense_attention_rows(q, k, v, [0, 9, 41]), ref[:, :, [0, 9, 41]], atol=1e-12)


def test_stage_r_is_blockwise_dense():
    q, k, v = _rand(GRID, seed=19)
    y = oracle.stage_r(q, k, v, GRID, 1)
    T, H, W = GRID
    blocks = lambda x: x.reshape(2 * T * H, 1, W, -1)
    ref = _sdpa(blocks(q), blocks(k), blocks(v)).reshape(y.shape)
    assert np.allclose(y, ref, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
def _mut_stage_order(q, k, v, grid, r_axes=1, tile=None):
    z = oracle.stage_l(q, k, v, grid, r_axes, tile)
    return oracle.stage_r(q, k, z, grid, r_axes)


def _mut_no_permutation(q, k, v, grid, r_axes=1, tile=None):
    # stage L over contiguous chunks of b1 tokens instead of stride-b2 sets
    y = oracle.stage_r(q, k, v, grid, r_axes)
    b1, b2 = oracle.block_sizes(grid, r_axes)
    groups = [np.arange(c * b1, (c + 1) * b1) for c in range(b2)]
    return oracle.monarch._per_head(
        lambda qq, kk, yy: oracle.group_softmax_attention(qq, kk, yy, groups), q, k, y)


def _mut_no_scale(q, k, v, grid, r_axes=1, tile=None):
    d = np.asarray(q).shape[-1]
    return oracle.monarch_attention(np.asarray(q) * math.sqrt(d), k, v, grid, r_axes, tile)


def _mut_drop_stage_r(q, k, v, grid, r_axes=1, tile=None):
    return oracle.stage_l(q, k, v, grid, r_axes, tile)


def _mut_tile_axes_swapped(q, k, v, grid, r_axes=1, tile=None):
    return oracle.monarch_attention(q, k, v, grid, r_axes, None if tile is None else (tile[1], tile[0]))


def _mut_keys_as_queries(q, k, v, grid, r_axes=1, tile=None):
    # transposed operand: logits k_n . q_m instead of q_n . k_m
    return oracle.monarch_attention(k, q, v, grid, r_axes, tile)


def _mut_sign(q, k, v, grid, r_axes=1, tile=None):
    return oracle.monarch_attention(-np.asarray(q), k, v, grid, r_axes, tile)


def _mut_stage_l_uses_y_as_keys(q, k, v, grid, r_axes=1, tile=None):
    y = oracle.stage_r(q, k, v, grid, r_axes)
    return oracle.stage_l(q, y, y, grid, r_axes, tile)


MUTANTS = [_mut_stage_order, _mut_no_permutation, _mut_no_scale, _mut_drop_stage_r,
           _mut_tile_axes_swapped, _mut_keys_as_queries, _mut_sign, _mut_stage_l_uses_y_as_keys]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_fails_a_pin(mutant):
    failed = []
    for pin in PINS:
        try:
            ok = pin(mutant)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, "no pin caught " + mutant.__name__
