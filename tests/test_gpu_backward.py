"""GPU parity of the backward pass (monarch_attn_bwd, bf16) against the fp64 backward oracle.

Gate (bf16 operands, fp32 accumulation, bf16 Y, dY and gradients): for each of
dq, dk, dv the relative L2 error ||g - g_ref|| / ||g_ref|| <= 1e-2, and every
element within 2e-2 * max|g_ref| of the reference. Each GPU gradient carries
the rounding of its bf16 operands (P, dS and the inputs as MFMA operands,
2^-9 relative each), of the bf16 intermediates Y and dY, and of its own bf16
output: a handful of independent 2^-9 roundings on any path, about 4e-3
relative in quadrature (measured: at most 3.7e-3 relative L2 and 7.5e-3 of
max|g_ref| over every case here), which the gates leave a factor of 2.5.
"""
import numpy as np
import pytest

from oracle import monarch_backward as mb
from workloads import WORKLOADS, make_qkv, to_bf16_f32

from parity_util import download, upload

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()


def run_bwd(q, k, v, do, grid, r_axes=1, tile=None, saved_y=False):
    """Forward then backward through the C ABI; returns (dq, dk, dv) as float64.
    saved_y: hand the forward's Y (its workspace) to the backward."""
    import torch
    import structured_attention_video_attn_amd as ma
    T, H, W = grid
    qd, kd, vd, dod = (upload(x, "bf16") for x in (q, k, v, do))
    B, h, N, d = qd.shape
    out = torch.empty_like(qd)
    tt, th = tile if tile else (0, 0)
    r = 1 if tile else r_axes
    nb = ma.ma_workspace_bytes(B, h, T, H, W, r, tt, th, d, ma.MA_BF16)
    ws = torch.empty(max(nb // 2, 1), dtype=torch.bfloat16, device="cuda")
    if tile:
        ma.monarch_attn_tiled_fwd(qd, kd, vd, out, ws, T, H, W, tt, th)
    else:
        ma.monarch_attn_fwd(qd, kd, vd, out, ws, T, H, W, r_axes)
    grads = [torch.full_like(qd, float("nan")) for _ in range(3)]
    nbw = ma.ma_bwd_workspace_bytes(B, h, T, H, W, r, tt, th, d, ma.MA_BF16)
    wsb = torch.full((nbw // 2,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = ws[:qd.numel()].view(qd.shape) if saved_y and nb > 0 else None
    ma.monarch_attn_bwd(qd, kd, vd, out, dod, *grads, wsb, T, H, W, r, tt, th, y=y)
    torch.cuda.synchronize()
    return tuple(download(g) for g in grads)


def check(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(g).all(), "%s %s: non-finite (an element was not written?)" % (label, name)
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        mx = float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-300))
        print("%s %s rel_l2=%.3e max/max|ref|=%.3e" % (label, name, rel, mx), flush=True)
        assert rel <= REL_L2, "%s %s rel_l2 %.3e" % (label, name, rel)
        assert mx <= MAX_REL, "%s %s max %.3e" % (label, name, mx)


def _randn(grid, heads, d, seed, n=4):
    rng = np.random.default_rng(seed)
    tok = grid[0] * grid[1] * grid[2]
    return [to_bf16_f32(rng.standard_normal((1, heads, tok, d), dtype=np.float32)) for _ in range(n)]


SMALL = [
    ((5, 27, 12), 1, None),       # stage L: 135 members = 3 key tiles (ragged); stage R groups of 12
    ((5, 27, 12), 1, (2, 5)),     # ragged boxes on both axes
    ((3, 7, 20), 2, None),        # stage R over 140-token frames (3 tiles), stage L groups of 3
    ((2, 3, 70), 1, None),        # stage R groups of 70 > 64, stage L of 6
    ((4, 5, 3), 0, None),         # b2 = 1: stage R trivial, one stage-L group of 60
    ((1, 1, 200), 3, None),       # one stage-R block of 200: dense attention
]


@pytest.mark.parametrize("d", [128, 64, 32, 16])
@pytest.mark.parametrize("grid,r_axes,tile", SMALL)
def test_backward_small(grid, r_axes, tile, d):
    q, k, v, do = _randn(grid, 2, d, seed=500 + d)
    got = run_bwd(q, k, v, do, grid, r_axes, tile)
    ref = mb.monarch_attention_backward(q, k, v, do, grid, r_axes=r_axes, tile=tile)
    check(got, ref, "bwd %s r=%d tile=%s d=%d" % (grid, r_axes, tile, d))


@pytest.mark.parametrize("d", [128, 32])
@pytest.mark.parametrize("grid,r_axes,tile", SMALL)
def test_backward_saved_y_same_bits(grid, r_axes, tile, d):
    # the forward's Y handed to the backward replaces the recomputed one bit for bit
    q, k, v, do = _randn(grid, 2, d, seed=600 + d)
    fresh = run_bwd(q, k, v, do, grid, r_axes, tile)
    saved = run_bwd(q, k, v, do, grid, r_axes, tile, saved_y=True)
    for name, a, b in zip(("dq", "dk", "dv"), fresh, saved):
        assert np.array_equal(a, b), "%s differs with the saved Y (%s r=%d tile=%s d=%d)" % (name, grid, r_axes, tile, d)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["chunk", "chunk_sharp"])
def test_backward_chunk(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl, heads=4)
    do = to_bf16_f32(np.random.default_rng(31).standard_normal(q.shape, dtype=np.float32))
    grid = (wl.T, wl.H, wl.W)
    check(run_bwd(q, k, v, do, grid), mb.monarch_attention_backward(q, k, v, do, grid), name + " bwd")
    # (3, 10) boxes: three per stage-L group at this 3-frame grid (the workload's own 3 x 30
    # tile spans whole groups here, where tiled and untiled coincide)
    ref_tiled = mb.monarch_attention_backward(q, k, v, do, grid, tile=(3, 10))
    check(run_bwd(q, k, v, do, grid, 1, (3, 10)), ref_tiled, name + " bwd tiled (3, 10)")
    check(run_bwd(q, k, v, do, grid, 1, (3, 10), saved_y=True), ref_tiled, name + " bwd tiled (3, 10), saved Y")


@pytest.mark.timeout(900)
def test_backward_full_two_heads():
    wl = WORKLOADS["full"]
    q, k, v = make_qkv(wl, heads=2)
    do = to_bf16_f32(np.random.default_rng(32).standard_normal(q.shape, dtype=np.float32))
    grid = (wl.T, wl.H, wl.W)
    check(run_bwd(q, k, v, do, grid), mb.monarch_attention_backward(q, k, v, do, grid), "full bwd (2 heads)")


@pytest.mark.timeout(900)
def test_backward_structured_tiled_two_heads():
    wl = WORKLOADS["structured"]
    q, k, v = make_qkv(wl, heads=2)
    do = to_bf16_f32(np.random.default_rng(34).standard_normal(q.shape, dtype=np.float32))
    grid = (wl.T, wl.H, wl.W)
    check(run_bwd(q, k, v, do, grid, 1, wl.tile), mb.monarch_attention_backward(q, k, v, do, grid, tile=wl.tile),
          "structured bwd tiled %s (2 heads)" % (wl.tile,))


@pytest.mark.timeout(900)
def test_backward_full_scale_all_heads_and_dv_sum():
    """All 12 heads at 21x30x52 compared whole with the backward oracle, and the
    oracle-free identity: summed over tokens, dV equals the summed dO (both factors
    are row-stochastic).

    Tolerance of the identity, from the bf16 roundings on the path (each a
    round-to-nearest with relative error uniform in +-2^-9, standard deviation
    2^-9/sqrt(3) of the rounded value, independent across elements): dv stored in
    bf16 (sum of dv^2), dY stored in bf16 and the stage-R weights rounded to bf16 as
    MFMA operands (each weighted by dY; per-row weight sums deviate by at most that
    relative amount, sum of P^2 <= 1), the stage-L weights rounded the same way
    (weighted by dO). The column sum's error then has standard deviation at most
    2^-9/sqrt(3) * sqrt(sum dv^2 + 2 sum dY^2 + sum dO^2); the gate is six of them."""
    wl = WORKLOADS["full"]
    q, k, v = make_qkv(wl)
    do = to_bf16_f32(np.random.default_rng(33).standard_normal(q.shape, dtype=np.float32))
    grid = (wl.T, wl.H, wl.W)
    got = run_bwd(q, k, v, do, grid)
    dq, dk, dv_ref, parts = mb.monarch_attention_backward(q, k, v, do, grid, return_parts=True)
    check(got, (dq, dk, dv_ref), "full bwd (12 heads)")
    dv = got[2]
    do64 = do.astype(np.float64)
    lhs, rhs = dv.sum(axis=2), do64.sum(axis=2)
    sigma = 2.0 ** -9 / np.sqrt(3.0) * np.sqrt((dv ** 2).sum(axis=2) + 2.0 * (parts["dy"] ** 2).sum(axis=2)
                                                + (do64 ** 2).sum(axis=2))
    worst = float((np.abs(lhs - rhs) / sigma).max())
    print("sum dV - sum dO: max |err| = %.3e, max |err| / sigma = %.2f" % (np.abs(lhs - rhs).max(), worst))
    assert worst <= 6.0
