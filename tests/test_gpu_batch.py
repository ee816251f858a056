"""GPU parity with batch > 1: every entry point against the fp64 oracle on [2, 3, N, d]
inputs, so that the (batch, head) slice arithmetic of each kernel is exercised with
both indices non-zero. Gates as in parity_util (bf16: max-abs 2e-2, G1, G2; fp32:
max-abs 1e-5) and, for the backward, those of test_gpu_backward.
"""
import numpy as np
import pytest

import oracle
from oracle import monarch_backward as mb
from oracle import monarch_causal as mc
from workloads import to_bf16_f32

from parity_util import (assert_bf16_parity, assert_f32_parity, download, run_dense, run_monarch, upload)

pytestmark = pytest.mark.gpu

B, HEADS = 2, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()


def _inputs(grid, d, seed, n=3, bf16=True):
    rng = np.random.default_rng(seed)
    tok = grid[0] * grid[1] * grid[2]
    xs = [rng.standard_normal((B, HEADS, tok, d), dtype=np.float32) for _ in range(n)]
    return [to_bf16_f32(x) for x in xs] if bf16 else xs


@pytest.mark.parametrize("grid,r_axes,tile,d", [
    ((4, 9, 20), 1, None, 128),    # stage R blocks of 20, stage L groups of 36
    ((3, 30, 12), 1, None, 64),    # stage L groups of 90 (streaming kernel)
    ((5, 4, 30), 2, None, 128),    # stage R over 120-token frames, stage L groups of 5
    ((6, 10, 8), 1, (4, 3), 32),   # ragged tiled boxes
])
def test_batch_forward_bf16(grid, r_axes, tile, d):
    q, k, v = _inputs(grid, d, seed=700 + d)
    got, _ = run_monarch(q, k, v, grid, "bf16", r_axes, tile)
    ref = oracle.monarch_attention(q, k, v, grid, r_axes=r_axes, tile=tile)
    assert_bf16_parity(got, ref, "batch %s r=%d tile=%s d=%d" % (grid, r_axes, tile, d))


def test_batch_forward_f32():
    grid = (2, 4, 4)
    q, k, v = _inputs(grid, 16, seed=710, bf16=False)
    for r_axes, tile in [(1, None), (2, None), (1, (1, 2))]:
        got, _ = run_monarch(q, k, v, grid, "f32", r_axes, tile)
        assert_f32_parity(got, oracle.monarch_attention(q, k, v, grid, r_axes=r_axes, tile=tile),
                          "batch f32 r=%d tile=%s" % (r_axes, tile))


def test_batch_dense():
    q, k, v = _inputs((1, 1, 300), 64, seed=720)
    assert_bf16_parity(run_dense(q, k, v, "bf16"), oracle.dense_attention(q, k, v), "batch dense")


def test_batch_causal_and_step():
    import torch
    import structured_attention_video_attn_amd as ma
    grid, ct = (6, 14, 10), 2   # chunks start at frames 0, 2, 4
    T, H, W = grid
    q, k, v = _inputs(grid, 128, seed=730)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    ws = torch.empty(ma.ma_workspace_bytes(B, HEADS, T, H, W) // 2, dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_causal_fwd(qd, kd, vd, out, ws, T, H, W, ct)
    torch.cuda.synchronize()
    assert_bf16_parity(download(out), mc.monarch_attention_causal(q, k, v, grid, ct), "batch causal")
    # the last chunk as one step, with the whole-sequence call's Y as the cache
    t0 = T - ct
    assert t0 % ct == 0
    y = ws[:qd.numel()].view(qd.shape).clone()
    fsz = H * W
    y[:, :, t0 * fsz:] = float("nan")
    o2 = torch.full_like(qd, float("nan"))
    ma.monarch_attn_chunk_fwd(qd, kd, vd, y, o2, T, H, W, t0, ct)
    torch.cuda.synchronize()
    assert torch.equal(o2[:, :, t0 * fsz:], out[:, :, t0 * fsz:])


def test_batch_backward():
    import torch
    import structured_attention_video_attn_amd as ma
    grid = (4, 18, 12)   # stage L groups of 72 (two-pass kernels), stage R groups of 12 (fused)
    T, H, W = grid
    q, k, v, do = _inputs(grid, 128, seed=740, n=4)
    qd, kd, vd, dod = (upload(x, "bf16") for x in (q, k, v, do))
    out = torch.empty_like(qd)
    ws = torch.empty(ma.ma_workspace_bytes(B, HEADS, T, H, W) // 2, dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_fwd(qd, kd, vd, out, ws, T, H, W)
    grads = [torch.full_like(qd, float("nan")) for _ in range(3)]
    wsb = torch.empty(ma.ma_bwd_workspace_bytes(B, HEADS, T, H, W) // 2, dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_bwd(qd, kd, vd, out, dod, *grads, wsb, T, H, W)
    torch.cuda.synchronize()
    ref = mb.monarch_attention_backward(q, k, v, do, grid)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        got = download(g)
        assert np.isfinite(got).all(), name
        rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
        mx = float(np.abs(got - r).max() / np.abs(r).max())
        assert rel <= 1e-2 and mx <= 2e-2, "batch backward %s rel %.3e max %.3e" % (name, rel, mx)
