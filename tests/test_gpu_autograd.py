"""GPU checks of the torch.autograd wrapper (structured_attention_video_attn_amd.autograd).

The wrapper only allocates and picks entry points, so its forward must equal
monarch_attn_fwd / monarch_attn_tiled_fwd bit for bit and its gradients must
equal monarch_attn_bwd's bit for bit; the gradients are also checked against
the fp64 backward oracle with the gates of test_gpu_backward (relative L2
1e-2, every element within 2e-2 of max|ref|).
"""
import numpy as np
import pytest

from oracle import monarch_backward as mb
from workloads import to_bf16_f32

from parity_util import download, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()


def _inputs(grid, heads, d, seed):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return [to_bf16_f32(rng.standard_normal((1, heads, n, d), dtype=np.float32)) for _ in range(4)]


@pytest.mark.parametrize("grid,r_axes,tile,d", [
    ((5, 27, 12), 1, None, 128),   # both stages, stage L over 135 members
    ((5, 27, 12), 1, (2, 5), 64),  # ragged tiled boxes
    ((3, 7, 20), 2, None, 32),     # frame blocks
    ((4, 5, 3), 0, None, 16),      # stage R the identity
])
def test_autograd_matches_entry_points_and_oracle(grid, r_axes, tile, d):
    import torch
    import structured_attention_video_attn_amd as ma
    from structured_attention_video_attn_amd.autograd import monarch_attention
    T, H, W = grid
    q, k, v, do = _inputs(grid, 2, d, seed=800 + d)
    qd, kd, vd, dod = (upload(x, "bf16") for x in (q, k, v, do))
    leaves = [x.clone().requires_grad_(True) for x in (qd, kd, vd)]
    out = monarch_attention(*leaves, T, H, W, r_axes=r_axes, tile=tile)
    out.backward(dod)
    torch.cuda.synchronize()
    # the entry points called directly (stage R recomputed by the backward)
    tt, th = tile if tile else (0, 0)
    r = 1 if tile else r_axes
    B_, h, N, _ = qd.shape
    ref_out = torch.empty_like(qd)
    nb = ma.ma_workspace_bytes(B_, h, T, H, W, r, tt, th, d, ma.MA_BF16)
    ws = torch.empty(max(nb // 2, 1), dtype=torch.bfloat16, device="cuda")
    if tile:
        ma.monarch_attn_tiled_fwd(qd, kd, vd, ref_out, ws, T, H, W, tt, th)
    else:
        ma.monarch_attn_fwd(qd, kd, vd, ref_out, ws, T, H, W, r_axes)
    grads = [torch.empty_like(qd) for _ in range(3)]
    wsb = torch.empty(ma.ma_bwd_workspace_bytes(B_, h, T, H, W, r, tt, th, d, ma.MA_BF16) // 2,
                      dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_bwd(qd, kd, vd, ref_out, dod, *grads, wsb, T, H, W, r, tt, th)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    for name, leaf, g in zip(("dq", "dk", "dv"), leaves, grads):
        assert torch.equal(leaf.grad, g), name
    ref = mb.monarch_attention_backward(q, k, v, do, grid, r_axes=r, tile=tile)
    for name, leaf, rg in zip(("dq", "dk", "dv"), leaves, ref):
        got = download(leaf.grad)
        rel = float(np.linalg.norm(got - rg) / np.linalg.norm(rg))
        mx = float(np.abs(got - rg).max() / np.abs(rg).max())
        assert rel <= 1e-2 and mx <= 2e-2, "%s rel %.3e max %.3e" % (name, rel, mx)


def test_autograd_rejects_fp32():
    import torch
    from structured_attention_video_attn_amd.autograd import monarch_attention
    x = torch.zeros(1, 1, 8, 16, device="cuda", dtype=torch.float32)
    with pytest.raises(TypeError):
        monarch_attention(x, x, x, 2, 2, 2)
