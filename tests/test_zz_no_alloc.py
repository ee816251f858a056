"""GPU test of monarch_attn_fwd_noalloc: the variant of monarch_attn_fwd whose
stage-R output Y lives in the library's fixed per-GPU buffer instead of a
caller's workspace. Through the C ABI, two calls in a row (the second with a
smaller problem, so it runs on whatever the first left in the buffer) must give
the same output as monarch_attn_fwd on the same inputs, and both must pass the
parity gates against the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_qkv, to_bf16_f32

from parity_util import assert_bf16_parity, assert_f32_parity, download, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import structured_attention_video_attn_amd as ma
    ma.load_library()


def _both(q, k, v, grid, dtype, r_axes=1):
    """(noalloc output, monarch_attn_fwd output) as float64, outputs NaN-poisoned."""
    import torch
    import structured_attention_video_attn_amd as ma
    T, H, W = grid
    qd, kd, vd = (upload(x, dtype) for x in (q, k, v))
    out_a = torch.full_like(qd, float("nan"))
    ma.monarch_attn_fwd_noalloc(qd, kd, vd, out_a, T, H, W, r_axes)
    torch.cuda.synchronize()
    B, h, N, d = qd.shape
    nb = ma.ma_workspace_bytes(B, h, T, H, W, r_axes, 0, 0, d, ma.MA_BF16 if dtype == "bf16" else ma.MA_F32)
    ws = torch.full((max(nb // qd.element_size(), 1),), float("nan"), dtype=qd.dtype, device="cuda")
    out_b = torch.full_like(qd, float("nan"))
    ma.monarch_attn_fwd(qd, kd, vd, out_b, ws if nb else None, T, H, W, r_axes)
    torch.cuda.synchronize()
    return download(out_a), download(out_b)


def test_noalloc_matches_workspace_entry_point_twice():
    # call 1: the 4680-token workload (12 heads, d128, bf16; Y 14.4 MB of the 128 MiB buffer)
    wl = WORKLOADS["chunk"]
    grid = (wl.T, wl.H, wl.W)
    q, k, v = make_qkv(wl)
    a, b = _both(q, k, v, grid, "bf16")
    assert np.array_equal(a, b), "noalloc differs from monarch_attn_fwd (4680 tokens)"
    assert_bf16_parity(a, oracle.monarch_attention(q, k, v, grid), "noalloc 3x30x52")

    # call 2, smaller: a ragged 5x27x12 grid, 2 heads, d64 (stage-L groups of 135)
    grid2 = (5, 27, 12)
    rng = np.random.default_rng(901)
    q2, k2, v2 = (to_bf16_f32(rng.standard_normal((1, 2, 5 * 27 * 12, 64), dtype=np.float32)) for _ in range(3))
    a2, b2 = _both(q2, k2, v2, grid2, "bf16")
    assert np.array_equal(a2, b2), "noalloc differs from monarch_attn_fwd (small, second call)"
    assert_bf16_parity(a2, oracle.monarch_attention(q2, k2, v2, grid2), "noalloc 5x27x12 d64")


def test_noalloc_fp32_and_frame_blocks():
    wl = WORKLOADS["tiny"]
    grid = (wl.T, wl.H, wl.W)
    q, k, v = make_qkv(wl)
    a, b = _both(q, k, v, grid, "f32")
    assert np.array_equal(a, b)
    assert_f32_parity(a, oracle.monarch_attention(q, k, v, grid), "noalloc tiny fp32")
    rng = np.random.default_rng(902)
    grid2 = (3, 7, 20)
    q2, k2, v2 = (to_bf16_f32(rng.standard_normal((1, 2, 420, 128), dtype=np.float32)) for _ in range(3))
    a2, b2 = _both(q2, k2, v2, grid2, "bf16", r_axes=2)
    assert np.array_equal(a2, b2)
    assert_bf16_parity(a2, oracle.monarch_attention(q2, k2, v2, grid2, r_axes=2), "noalloc r_axes=2")


def test_noalloc_rejects_oversized_problem():
    import torch
    import structured_attention_video_attn_amd as ma
    # 24 heads at 21x30x52, d128, bf16: Y is 201 MB, more than the 128 MiB buffer
    q = torch.empty((1, 24, 32760, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ma.MonarchAttnError, match="MA_ERR_SCRATCH"):
        ma.monarch_attn_fwd_noalloc(q, q, q, out, 21, 30, 52)
