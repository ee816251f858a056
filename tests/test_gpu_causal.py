"""GPU parity of the chunk-causal forms (monarch_attn_causal_fwd, monarch_attn_chunk_fwd)
against the fp64 chunk-causal oracle, through the C ABI.

Gates: those of the bf16 forward (parity_util: max-abs 2e-2, G1 1e-2, G2 0.1).
Besides the oracle, the step form must reproduce the whole-sequence form
bitwise chunk by chunk (the same kernels see the same inputs, and every wave
holds the same 32 queries), and chunk_t >= T must reproduce monarch_attn_fwd
bitwise. Outputs and the Y cache are NaN-poisoned before each call; a step
must leave every frame outside its chunk untouched.
"""
import numpy as np
import pytest

import oracle
from oracle import monarch_causal as mc
from workloads import CAUSAL_CHUNK_T, WORKLOADS, make_qkv, to_bf16_f32

from parity_util import assert_bf16_parity, download, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()


def _randn(grid, heads, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    n = grid[0] * grid[1] * grid[2]
    return [to_bf16_f32(scale * rng.standard_normal((1, heads, n, d), dtype=np.float32)) for _ in range(3)]


def run_causal(qd, kd, vd, grid, chunk_t, r_axes=1):
    import torch
    import structured_attention_video_attn_amd as ma
    T, H, W = grid
    B, h, N, d = qd.shape
    out = torch.full_like(qd, float("nan"))
    nb = ma.ma_workspace_bytes(B, h, T, H, W, r_axes, 0, 0, d, ma.MA_BF16)
    ws = torch.full((max(nb // 2, 1),), float("nan"), dtype=torch.bfloat16, device="cuda") if nb else None
    ma.monarch_attn_causal_fwd(qd, kd, vd, out, ws, T, H, W, chunk_t, r_axes)
    torch.cuda.synchronize()
    return out


def run_steps(qd, kd, vd, grid, chunk_t, r_axes=1):
    """Every chunk in order through monarch_attn_chunk_fwd, with one growing Y cache."""
    import torch
    import structured_attention_video_attn_amd as ma
    T, H, W = grid
    fsz = H * W
    out = torch.full_like(qd, float("nan"))
    y = torch.full_like(qd, float("nan")) if r_axes != 0 else None
    for t0 in range(0, T, chunk_t):
        n = min(chunk_t, T - t0)
        before = out.clone()
        ma.monarch_attn_chunk_fwd(qd, kd, vd, y, out, T, H, W, t0, n, r_axes)
        torch.cuda.synchronize()
        # frames outside the chunk are untouched
        lo, hi = t0 * fsz, (t0 + n) * fsz
        assert torch.equal(torch.isnan(out[:, :, :lo]), torch.isnan(before[:, :, :lo]))
        assert bool(torch.isnan(out[:, :, hi:]).all())
        if y is not None:
            assert bool(torch.isnan(y[:, :, hi:]).all())
    return out


SMALL = [
    ((5, 27, 12), 2, 1, 128),    # 2-frame chunks; stage-L groups of 135 (three key tiles), ragged last chunk
    ((6, 14, 20), 3, 1, 64),     # spans of 42 members
    ((7, 3, 40), 1, 2, 128),     # frame-level causality, stage-L groups of 7
    ((4, 9, 8), 2, 0, 32),       # r_axes 0: stage L over every token, spans of 144
    ((9, 10, 6), 4, 1, 16),      # spans of 40, ragged last chunk of 1 frame
]


@pytest.mark.parametrize("grid,chunk_t,r_axes,d", SMALL)
def test_causal_small(grid, chunk_t, r_axes, d):
    q, k, v = _randn(grid, 2, d, seed=300 + d + chunk_t)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    got = run_causal(qd, kd, vd, grid, chunk_t, r_axes)
    ref = mc.monarch_attention_causal(q, k, v, grid, chunk_t, r_axes)
    assert_bf16_parity(download(got), ref, "causal %s ct=%d r=%d d=%d" % (grid, chunk_t, r_axes, d))
    steps = run_steps(qd, kd, vd, grid, chunk_t, r_axes)
    import torch
    assert torch.equal(steps, got), "chunk steps differ from the whole-sequence form"


def test_chunk_at_least_t_is_bidirectional():
    import torch
    import structured_attention_video_attn_amd as ma
    grid = (4, 30, 20)   # stage-L groups of 120: both forms take the streaming kernel
    q, k, v = _randn(grid, 2, 128, seed=41)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    T, H, W = grid
    out = torch.empty_like(qd)
    ws = torch.empty(ma.ma_workspace_bytes(1, 2, T, H, W) // 2, dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_fwd(qd, kd, vd, out, ws, T, H, W)
    for ct in (T, T + 5):
        assert torch.equal(run_causal(qd, kd, vd, grid, ct), out)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["full", "full_sharp"])
def test_causal_full_scale(name):
    wl = WORKLOADS[name]
    grid = (wl.T, wl.H, wl.W)
    q, k, v = make_qkv(wl)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    got = run_causal(qd, kd, vd, grid, CAUSAL_CHUNK_T)
    ref = mc.monarch_attention_causal(q, k, v, grid, CAUSAL_CHUNK_T)
    assert_bf16_parity(download(got), ref, name + " causal")


@pytest.mark.timeout(600)
def test_chunk_step_with_cache_full_scale():
    """The last 3-frame chunk of the 21-frame workload, Y cache from the GPU's own stage R."""
    import torch
    import structured_attention_video_attn_amd as ma
    wl = WORKLOADS["full"]
    grid = (wl.T, wl.H, wl.W)
    T, H, W = grid
    fsz = H * W
    t0, ct = T - CAUSAL_CHUNK_T, CAUSAL_CHUNK_T
    q, k, v = make_qkv(wl)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    y = torch.empty_like(qd)
    ma.ma_stage_r_fwd(qd, kd, vd, y, T, H, W)     # the cache: Y of every frame
    y[:, :, t0 * fsz:] = float("nan")             # the chunk's Y must be recomputed
    out = torch.full_like(qd, float("nan"))
    ma.monarch_attn_chunk_fwd(qd, kd, vd, y, out, T, H, W, t0, ct)
    torch.cuda.synchronize()
    y_ref, o_ref = mc.monarch_attention_chunk_step(q, k, v, oracle.stage_r(q, k, v, grid), grid, t0, ct)
    assert_bf16_parity(download(y[:, :, t0 * fsz:]), y_ref, "chunk step Y")
    assert_bf16_parity(download(out[:, :, t0 * fsz:]), o_ref, "chunk step O")
    assert bool(torch.isnan(out[:, :, :t0 * fsz]).all())


def test_first_chunk_equals_monarch_of_its_frames():
    import torch
    import structured_attention_video_attn_amd as ma
    grid = (5, 30, 52)
    T, H, W = grid
    ct = 3
    q, k, v = _randn(grid, 3, 128, seed=51, scale=1.0 / 128 ** 0.25)
    qd, kd, vd = (upload(x, "bf16") for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    y = torch.full_like(qd, float("nan"))
    ma.monarch_attn_chunk_fwd(qd, kd, vd, y, out, T, H, W, 0, ct)
    n = ct * H * W
    sub = [x[:, :, :n].contiguous() for x in (qd, kd, vd)]
    o2 = torch.empty_like(sub[0])
    ws = torch.empty(ma.ma_workspace_bytes(1, 3, ct, H, W) // 2, dtype=torch.bfloat16, device="cuda")
    ma.monarch_attn_fwd(*sub, o2, ws, ct, H, W)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, :n], o2)
    assert torch.equal(y[:, :, :n], ws[:o2.numel()].view(o2.shape))
