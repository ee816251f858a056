"""Pins for the chunk-causal oracle (oracle/monarch_causal.py): checks that do not
use its masked stage-L formula.

Each pin takes an implementation ``g(q, k, v, grid, chunk_t, r_axes) -> O`` of the
whole-sequence chunk-causal operator, so that the same checks also run against
broken copies (planted mistakes, CPU only).

Sources of truth:
* the prefix property of the reading: the rows of chunk c equal the
  bidirectional Monarch operator (the pinned forward oracle) over the grid of
  frames [0, (c+1) chunk_t), at those rows;
* chunk_t >= T: the bidirectional operator itself;
* r_axes = 2, chunk_t = 1 (stage-L groups are one token per frame): stage L is
  textbook causal attention over frames at each (h, w), i.e. torch's float64
  ``scaled_dot_product_attention(..., is_causal=True)`` on Y;
* causality: changing every input of a later chunk leaves earlier chunks'
  outputs unchanged, while changing an input inside the same chunk does not;
* the single-step form agrees with the whole-sequence form chunk by chunk.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import monarch_causal as mc


def _rand(grid, d=8, heads=2, seed=21):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((1, heads, n, d)) for _ in range(3)]


def _oracle(q, k, v, grid, chunk_t, r_axes=1):
    return mc.monarch_attention_causal(q, k, v, grid, chunk_t, r_axes)


CASES = [((5, 3, 4), 2, 1), ((4, 2, 3), 1, 1), ((6, 2, 2), 3, 2), ((3, 2, 3), 1, 0), ((5, 2, 3), 2, 0)]


def pin_prefix(g):
    ok = True
    for grid, ct, r in CASES:
        T, H, W = grid
        q, k, v = _rand(grid, seed=22 + T)
        o = g(q, k, v, grid, ct, r)
        fsz = H * W
        for c in range((T + ct - 1) // ct):
            t_end = min(T, (c + 1) * ct)
            sub = (t_end, H, W)
            ref = oracle.monarch_attention(q[:, :, :t_end * fsz], k[:, :, :t_end * fsz], v[:, :, :t_end * fsz],
                                           sub, r_axes=r)
            lo = c * ct * fsz
            ok &= np.allclose(o[:, :, lo:t_end * fsz], ref[:, :, lo:], rtol=0, atol=1e-12)
    return ok


def pin_whole_chunk_is_bidirectional(g):
    ok = True
    for grid, _, r in CASES:
        q, k, v = _rand(grid, seed=31)
        ref = oracle.monarch_attention(q, k, v, grid, r_axes=r)
        for ct in (grid[0], grid[0] + 3):
            ok &= np.allclose(g(q, k, v, grid, ct, r), ref, rtol=0, atol=1e-12)
    return ok


def pin_frame_causal_sdpa(g):
    grid = (6, 2, 3)
    T, H, W = grid
    q, k, v = _rand(grid, seed=41)
    y = oracle.stage_r(q, k, v, grid, r_axes=2)
    o = g(q, k, v, grid, 1, 2)
    # stage-L group of position p = h*W + w is the tokens t*H*W + p over frames t
    ok = True
    for pos in range(H * W):
        idx = np.arange(T) * H * W + pos
        qt, kt, yt = (torch.from_numpy(np.ascontiguousarray(x[:, :, idx])) for x in (q, k, y))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, yt, is_causal=True).numpy()
        ok &= np.allclose(o[:, :, idx], ref, rtol=0, atol=1e-12)
    return ok


def pin_causality(g):
    ok = True
    for grid, ct, r in CASES:
        T, H, W = grid
        fsz = H * W
        q, k, v = _rand(grid, seed=51)
        base = g(q, k, v, grid, ct, r)
        rng = np.random.default_rng(52)
        for c in range(1, (T + ct - 1) // ct):
            lo = c * ct * fsz
            q2, k2, v2 = (x.copy() for x in (q, k, v))
            for x in (q2, k2, v2):
                x[:, :, lo:] = rng.standard_normal(x[:, :, lo:].shape)
            other = g(q2, k2, v2, grid, ct, r)
            ok &= np.allclose(other[:, :, :lo], base[:, :, :lo], rtol=0, atol=1e-12)   # past unchanged
            ok &= not np.allclose(other[:, :, lo:lo + fsz], base[:, :, lo:lo + fsz], atol=1e-6)
        # a key/value change inside the first chunk's last frame must reach its first frame
        if ct > 1:
            t_last = min(T, ct) - 1
            k3, v3 = k.copy(), v.copy()
            k3[:, :, t_last * fsz:(t_last + 1) * fsz] += 1.0
            v3[:, :, t_last * fsz:(t_last + 1) * fsz] += 1.0
            other = g(q, k3, v3, grid, ct, r)
            ok &= not np.allclose(other[:, :, :fsz], base[:, :, :fsz], atol=1e-6)
    return ok


def pin_step_matches_sequence(g):
    ok = True
    for grid, ct, r in CASES:
        T, H, W = grid
        fsz = H * W
        q, k, v = _rand(grid, seed=61)
        whole = g(q, k, v, grid, ct, r)
        y_cache = np.full(q.shape, np.nan)
        for t0 in range(0, T, ct):
            n = min(ct, T - t0)   # the last chunk may be shorter
            yc, oc = mc.monarch_attention_chunk_step(q, k, v, y_cache, grid, t0, n, r)
            y_cache[:, :, t0 * fsz:(t0 + n) * fsz] = yc
            ok &= np.allclose(oc, whole[:, :, t0 * fsz:(t0 + n) * fsz], rtol=0, atol=1e-12)
    return ok


PINS = [pin_prefix, pin_whole_chunk_is_bidirectional, pin_frame_causal_sdpa, pin_causality,
        pin_step_matches_sequence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_causal_oracle_passes_pin(pin):
    assert pin(_oracle)


def test_step_reads_no_later_frame():
    # frames after the chunk may hold anything: the step's result must not change
    grid, ct, r = (5, 3, 4), 2, 1
    fsz = 12
    q, k, v = _rand(grid, seed=71)
    y_cache = oracle.stage_r(q, k, v, grid, r_axes=r)
    yc, oc = mc.monarch_attention_chunk_step(q, k, v, y_cache, grid, 1, ct, r)
    q2, k2, v2, y2 = (x.copy() for x in (q, k, v, y_cache))
    for x in (q2, k2, v2, y2):
        x[:, :, 3 * fsz:] = 1e6
    y2[:, :, fsz:3 * fsz] = -7.0   # the chunk's own Y is recomputed, not read
    yc2, oc2 = mc.monarch_attention_chunk_step(q2, k2, v2, y2, grid, 1, ct, r)
    assert np.allclose(oc, oc2, atol=1e-12) and np.allclose(yc, yc2, atol=1e-12)


def test_rejects_stage_r_across_frames():
    q, k, v = _rand((2, 2, 2))
    with pytest.raises(ValueError):
        mc.monarch_attention_causal(q, k, v, (2, 2, 2), 1, r_axes=3)


# ---------------------------------------------------------------- planted mistakes
def _mut_strict(q, k, v, grid, chunk_t, r_axes=1):
    # keys of earlier chunks only (own chunk excluded), own token kept so rows are not empty
    y = oracle.stage_r(q, k, v, grid, r_axes)
    T, H, W = grid
    s = 1.0 / math.sqrt(q.shape[-1])
    ch = mc.member_frames(grid) // chunk_t
    out = np.empty_like(y)
    for g in oracle.stage_l_groups(grid, r_axes):
        for n in g:
            keys = [m for m in g if ch[m] < ch[n] or m == n]
            for b in range(q.shape[0]):
                for h in range(q.shape[1]):
                    lg = s * (k[b, h, keys] @ q[b, h, n])
                    p = np.exp(lg - lg.max())
                    out[b, h, n] = (p / p.sum()) @ y[b, h, keys]
    return out


def _mut_frame_granularity(q, k, v, grid, chunk_t, r_axes=1):
    return mc.monarch_attention_causal(q, k, v, grid, 1, r_axes)


def _mut_noncausal(q, k, v, grid, chunk_t, r_axes=1):
    return oracle.monarch_attention(q, k, v, grid, r_axes=r_axes)


def _mut_future(q, k, v, grid, chunk_t, r_axes=1):
    # anti-causal: keys of the own and later chunks
    T = grid[0]
    qr, kr, vr = (_reverse_frames(x, grid) for x in (q, k, v))
    o = mc.monarch_attention_causal(qr, kr, vr, grid, chunk_t, r_axes)
    return _reverse_frames(o, grid) if T % chunk_t == 0 else o


def _reverse_frames(x, grid):
    T, H, W = grid
    return np.ascontiguousarray(x.reshape(x.shape[0], x.shape[1], T, H * W, -1)[:, :, ::-1]).reshape(x.shape)


def _mut_v_as_values(q, k, v, grid, chunk_t, r_axes=1):
    # stage L takes V instead of Y
    return mc.causal_stage_l(q, k, v, grid, chunk_t, r_axes)


MUTANTS = [_mut_strict, _mut_frame_granularity, _mut_noncausal, _mut_future, _mut_v_as_values]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_causal_mistake_fails_a_pin(mutant):
    failed = []
    for pin in PINS:
        try:
            ok = pin(mutant)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, "no pin catches %s" % mutant.__name__
