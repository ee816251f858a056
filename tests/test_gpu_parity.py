"""GPU parity: the HIP library through its C ABI against the fp64 CPU oracle.

Sizes: the oracle covers the small cases and the 4680- and 32760-token
workloads whole; at 126360 tokens it covers four seeded heads whole and
seeded rows of every head.
bf16 cases pass the max-abs 2e-2 gate plus the relative gates G1/G2 of
parity_util; fp32 cases pass max-abs 1e-5.
"""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_qkv

from parity_util import (assert_bf16_parity, assert_f32_parity, run_dense, run_monarch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()   # raises if the HIP library is not built
    torch.manual_seed(0)


def _grid(wl):
    return (wl.T, wl.H, wl.W)


def _randn(grid, heads, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    from workloads import to_bf16_f32
    return [to_bf16_f32(scale * rng.standard_normal((1, heads, n, d), dtype=np.float32)) for _ in range(3)]


# ------------------------------------------------------------------ fp32 path, tiny grid
TINY_SPECS = [(1, None), (0, None), (2, None), (3, None), (1, (1, 2)), (1, (2, 2)), (1, (1, 1)),
              (1, (2, 4)), (1, (1, 3))]


@pytest.mark.parametrize("r_axes,tile", TINY_SPECS)
def test_tiny_f32(r_axes, tile):
    wl = WORKLOADS["tiny"]
    q, k, v = make_qkv(wl)
    got, _ = run_monarch(q, k, v, _grid(wl), "f32", r_axes, tile)
    ref = oracle.monarch_attention(q, k, v, _grid(wl), r_axes=r_axes, tile=tile)
    assert_f32_parity(got, ref, "tiny r=%d tile=%s" % (r_axes, tile))


def test_tiny_f32_single_block_is_dense():
    wl = WORKLOADS["tiny"]
    q, k, v = make_qkv(wl)
    ref = oracle.dense_attention(q, k, v)
    got, _ = run_monarch(q, k, v, _grid(wl), "f32", 3, None)
    assert_f32_parity(got, ref, "tiny single block")
    assert_f32_parity(run_dense(q, k, v, "f32"), ref, "tiny dense_attn_fwd")


# ------------------------------------------------------------------ small ragged shapes, all head dims
SMALL = [
    ((5, 27, 12), 1, None),       # stage L: 135 members = 3 key tiles (ragged), 2 query tiles
    ((5, 27, 12), 1, (2, 5)),     # ragged boxes on both axes
    ((3, 7, 20), 2, None),        # stage R over 140-token frames: streaming over 3 key tiles
    ((2, 3, 70), 1, None),        # stage R block of 70 > 64 keys, stage L of 6
    ((4, 5, 3), 0, None),         # one stage-L group of all 60 tokens
    ((1, 1, 200), 3, None),       # one stage-R block of 200 tokens
]


@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("grid,r_axes,tile", SMALL)
def test_small_bf16(grid, r_axes, tile, d):
    q, k, v = _randn(grid, 2, d, seed=100 + d)
    got, _ = run_monarch(q, k, v, grid, "bf16", r_axes, tile)
    ref = oracle.monarch_attention(q, k, v, grid, r_axes=r_axes, tile=tile)
    assert_bf16_parity(got, ref, "small bf16 %s r=%d tile=%s d=%d" % (grid, r_axes, tile, d))


# Stage-L groups of T*H = 65, 80, 96 and 97 members: the last key tile holds 1, 16 and 32
# keys (its second 32-key block is empty, so the streaming kernel runs that tile in its
# half form) and 33 keys (the full form), at every head dim the streaming kernel serves.
HALF_TILE_GRIDS = [(5, 13, 3), (4, 20, 3), (4, 24, 3), (1, 97, 3)]


@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("grid", HALF_TILE_GRIDS)
def test_last_key_tile_boundary(grid, d):
    q, k, v = _randn(grid, 2, d, seed=400 + d + grid[0] * grid[1])
    got, _ = run_monarch(q, k, v, grid, "bf16", 1, None)
    ref = oracle.monarch_attention(q, k, v, grid)
    keys_in_last = grid[0] * grid[1] - 64
    assert_bf16_parity(got, ref, "last key tile of %d keys %s d=%d" % (keys_in_last, grid, d))


@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("grid,r_axes,tile", SMALL)
def test_small_f32(grid, r_axes, tile, d):
    q, k, v = _randn(grid, 2, d, seed=200 + d)
    got, _ = run_monarch(q, k, v, grid, "f32", r_axes, tile)
    ref = oracle.monarch_attention(q, k, v, grid, r_axes=r_axes, tile=tile)
    assert_f32_parity(got, ref, "small f32 %s r=%d tile=%s d=%d" % (grid, r_axes, tile, d))


@pytest.mark.parametrize("n", [1, 63, 64, 65, 300])
def test_dense_small(n):
    q, k, v = _randn((1, 1, n), 3, 64, seed=300 + n)
    ref = oracle.dense_attention(q, k, v)
    assert_bf16_parity(run_dense(q, k, v, "bf16"), ref, "dense n=%d" % n, check_g2=n > 1)
    assert_f32_parity(run_dense(q, k, v, "f32"), ref, "dense f32 n=%d" % n)


# ------------------------------------------------------------------ video workloads
@pytest.mark.parametrize("name", ["chunk", "chunk_sharp"])
def test_chunk(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    got, y = run_monarch(q, k, v, _grid(wl), "bf16")
    ref, yref = oracle.monarch_attention(q, k, v, _grid(wl), return_y=True)
    assert_bf16_parity(y, yref, name + " stage R (workspace Y)")
    assert_bf16_parity(got, ref, name + " monarch")
    got_t, _ = run_monarch(q, k, v, _grid(wl), "bf16", 1, wl.tile)
    ref_t = oracle.monarch_attention(q, k, v, _grid(wl), tile=wl.tile)
    assert_bf16_parity(got_t, ref_t, name + " tiled %s" % (wl.tile,))


@pytest.mark.parametrize("name", ["chunk", "chunk_sharp"])
def test_chunk_f32(name):
    """The fp32 path (matrix-core kernel at head_dim 128) at the one-chunk workload; the
    sharp variant's peaked softmax exercises the running-max rescale."""
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    got, y = run_monarch(q, k, v, _grid(wl), "f32")
    ref, yref = oracle.monarch_attention(q, k, v, _grid(wl), return_y=True)
    assert_f32_parity(y, yref, name + " f32 stage R (workspace Y)")
    assert_f32_parity(got, ref, name + " f32 monarch")
    got_t, _ = run_monarch(q, k, v, _grid(wl), "f32", 1, wl.tile)
    assert_f32_parity(got_t, oracle.monarch_attention(q, k, v, _grid(wl), tile=wl.tile),
                      name + " f32 tiled %s" % (wl.tile,))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["full", "full_sharp"])
def test_full(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    got, _ = run_monarch(q, k, v, _grid(wl), "bf16")
    ref = oracle.monarch_attention(q, k, v, _grid(wl))
    assert_bf16_parity(got, ref, name + " monarch")


@pytest.mark.timeout(900)
def test_structured_tiled():
    wl = WORKLOADS["structured"]
    q, k, v = make_qkv(wl)
    got, _ = run_monarch(q, k, v, _grid(wl), "bf16", 1, wl.tile)
    ref = oracle.monarch_attention(q, k, v, _grid(wl), tile=wl.tile)
    assert_bf16_parity(got, ref, "structured tiled %s" % (wl.tile,))
    got_u, _ = run_monarch(q, k, v, _grid(wl), "bf16")
    ref_u = oracle.monarch_attention(q, k, v, _grid(wl))
    assert_bf16_parity(got_u, ref_u, "structured untiled")


@pytest.mark.timeout(900)
def test_long_whole_heads():
    """126360 tokens, 16 heads: four seeded heads compared whole (every output row),
    untiled (stage-L groups of 2430 over 38 key tiles) and in 9 x 30 tiles (boxes of 270),
    plus seeded rows of every head through the row-wise oracle."""
    wl = WORKLOADS["long"]
    q, k, v = make_qkv(wl)
    rng = np.random.default_rng(44)
    heads = sorted(rng.choice(wl.heads, size=4, replace=False).tolist())
    rows = sorted(rng.choice(wl.n_tokens, size=4, replace=False).tolist()) + [0, wl.n_tokens - 1]
    qh, kh, vh = (np.ascontiguousarray(x[:, heads]) for x in (q, k, v))
    for tile in (None, wl.tile):
        got, _ = run_monarch(q, k, v, _grid(wl), "bf16", 1, tile)
        assert np.isfinite(got).all()
        ref = oracle.monarch_attention(qh, kh, vh, _grid(wl), tile=tile)
        assert_bf16_parity(got[:, heads], ref, "long tile=%s (heads %s whole)" % (tile, heads))
        ref_rows = oracle.monarch_attention_rows(q, k, v, _grid(wl), rows, tile=tile)
        assert_bf16_parity(got[:, :, rows], ref_rows, "long tile=%s (16 heads x %d rows)" % (tile, len(rows)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["chunk", "full"])
def test_dense_comparator(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    got = run_dense(q, k, v, "bf16")
    assert np.isfinite(got).all()
    rows = sorted(np.random.default_rng(45).choice(wl.n_tokens, size=256, replace=False).tolist())
    ref = oracle.dense_attention_rows(q, k, v, rows)
    assert_bf16_parity(got[:, :, rows], ref, name + " dense (256 rows/head)")


# ------------------------------------------------------------------ frame-aligned blocks (r_axes = 2)
# b2 = H*W = 1560 spatial tokens per stage-R block, b1 = T frames per stage-L group: stage R runs
# the streaming kernel (25 key tiles per block), stage L the short-group kernel.
@pytest.mark.timeout(600)
def test_frame_blocks_chunk():
    wl = WORKLOADS["chunk"]
    q, k, v = make_qkv(wl)
    got, y = run_monarch(q, k, v, _grid(wl), "bf16", 2)
    ref, yref = oracle.monarch_attention(q, k, v, _grid(wl), r_axes=2, return_y=True)
    assert_bf16_parity(y, yref, "chunk r_axes=2 stage R (workspace Y)")
    assert_bf16_parity(got, ref, "chunk r_axes=2")


@pytest.mark.timeout(600)
def test_frame_blocks_full_whole_heads():
    """r_axes = 2 at 32760 tokens: three seeded heads compared whole (stage R over 21
    frames of 1560 tokens, 25 key tiles each; stage L over groups of 21)."""
    wl = WORKLOADS["full"]
    q, k, v = make_qkv(wl)
    got, _ = run_monarch(q, k, v, _grid(wl), "bf16", 2)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(46)
    heads = sorted(rng.choice(wl.heads, size=3, replace=False).tolist())
    qh, kh, vh = (np.ascontiguousarray(x[:, heads]) for x in (q, k, v))
    ref = oracle.monarch_attention(qh, kh, vh, _grid(wl), r_axes=2)
    assert_bf16_parity(got[:, heads], ref, "full r_axes=2 (heads %s whole)" % (heads,))


# ------------------------------------------------------------------ closed forms at full scale
@pytest.mark.timeout(600)
def test_closed_forms_full_scale():
    wl = WORKLOADS["full"]
    q, k, v = make_qkv(wl)
    grid = _grid(wl)
    ones = np.ones_like(v)
    for tile in (None, wl.tile):
        got, _ = run_monarch(q, k, ones, grid, "bf16", 1, tile)
        assert np.abs(got - 1.0).max() <= 1e-2, "V = 1 must give 1 (tile %s)" % (tile,)
    zeros = np.zeros_like(q)
    got, _ = run_monarch(zeros, k, v, grid, "bf16")
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)
    assert np.abs(got - mean).max() <= 2e-3
    got, _ = run_monarch(zeros, k, v, grid, "bf16", 1, wl.tile)
    T, H, W = grid
    tt, th = wl.tile
    vg = v.astype(np.float64).reshape(1, wl.heads, T // tt, tt, H // th, th, W, -1)
    box = vg.mean(axis=(3, 5, 6), keepdims=True)
    exp = np.broadcast_to(box, vg.shape).reshape(got.shape)
    assert np.abs(got - exp).max() <= 1e-2


@pytest.mark.timeout(600)
def test_deterministic_and_permutation_equivariant():
    wl = WORKLOADS["full_sharp"]
    q, k, v = make_qkv(wl, heads=4)
    grid = _grid(wl)
    a, _ = run_monarch(q, k, v, grid, "bf16")
    b, _ = run_monarch(q, k, v, grid, "bf16")
    assert np.array_equal(a, b), "two identical calls differ"
    T, H, W = grid

    def flip_w(x):
        return np.ascontiguousarray(x.reshape(1, 4, T, H, W, -1)[:, :, :, :, ::-1]).reshape(x.shape)

    c, _ = run_monarch(flip_w(q), flip_w(k), flip_w(v), grid, "bf16")
    assert np.abs(c - flip_w(a)).max() <= 1e-2
