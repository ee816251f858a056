"""Helpers for GPU-vs-oracle parity tests: device upload, calls through the C ABI, gates.

Gates for the bf16 path (inputs bf16, fp32 accumulation, bf16 intermediate and output):
  * max-abs error <= 2e-2 against the fp64 oracle;
  * G1: relative L2 error ||O - O_ref|| / ||O_ref|| <= 1e-2;
  * G2: ||O - O_ref|| / ||O_ref - mean_ref|| <= 0.1, with mean_ref the head's
    token-mean output, so that an output which ignores Q and K (nearly flat
    softmax) cannot pass by being close to the mean.
The fp32 path: max-abs error <= 1e-5.
"""
import numpy as np

MAX_ABS_BF16 = 2e-2
MAX_ABS_F32 = 1e-5
G1_MAX = 1e-2
G2_MAX = 0.1


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def upload(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def download(t):
    import torch
    return t.to(torch.float32).cpu().numpy().astype(np.float64)


def run_monarch(q, k, v, grid, dtype="bf16", r_axes=1, tile=None, poison=True):
    """Run monarch_attn_fwd / monarch_attn_tiled_fwd; returns (O, Y-workspace or None) as float64."""
    import torch
    import structured_attention_video_attn_amd as ma
    T, H, W = grid
    qd, kd, vd = (upload(x, dtype) for x in (q, k, v))
    out = torch.empty_like(qd)
    if poison:
        out.fill_(float("nan"))
    B, h, N, d = qd.shape
    code = ma.MA_BF16 if dtype == "bf16" else ma.MA_F32
    tt, th = tile if tile else (0, 0)
    nbytes = ma.ma_workspace_bytes(B, h, T, H, W, r_axes if tile is None else 1, tt, th, d, code)
    ws = None
    if nbytes:
        ws = torch.empty(nbytes // qd.element_size(), dtype=qd.dtype, device="cuda")
        if poison:
            ws.fill_(float("nan"))
    if tile is None:
        ma.monarch_attn_fwd(qd, kd, vd, out, ws, T, H, W, r_axes)
    else:
        ma.monarch_attn_tiled_fwd(qd, kd, vd, out, ws, T, H, W, tile[0], tile[1])
    torch.cuda.synchronize()
    return download(out), (None if ws is None else download(ws[:qd.numel()].view(qd.shape)))


def run_dense(q, k, v, dtype="bf16"):
    import torch
    import structured_attention_video_attn_amd as ma
    qd, kd, vd = (upload(x, dtype) for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    ma.dense_attn_fwd(qd, kd, vd, out)
    torch.cuda.synchronize()
    return download(out)


def errors(got, ref):
    """(max-abs, G1, G2) of got against ref, both [B, h, n, d]."""
    diff = got - ref
    max_abs = float(np.nanmax(np.abs(diff))) if np.isfinite(got).all() else float("inf")
    g1 = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    centered = ref - ref.mean(axis=2, keepdims=True)
    g2 = float(np.linalg.norm(diff) / max(np.linalg.norm(centered), 1e-300))
    return max_abs, g1, g2


def assert_bf16_parity(got, ref, label="", check_g2=True):
    assert np.isfinite(got).all(), label + ": non-finite output (an element was not written?)"
    max_abs, g1, g2 = errors(got, ref)
    print("%s max_abs=%.3e G1=%.3e G2=%.3e" % (label, max_abs, g1, g2), flush=True)
    assert max_abs <= MAX_ABS_BF16, label
    assert g1 <= G1_MAX, label
    if check_g2:
        assert g2 <= G2_MAX, label


def assert_f32_parity(got, ref, label=""):
    assert np.isfinite(got).all(), label + ": non-finite output"
    max_abs = float(np.abs(got - ref).max())
    print("%s max_abs=%.3e" % (label, max_abs), flush=True)
    assert max_abs <= MAX_ABS_F32, label
