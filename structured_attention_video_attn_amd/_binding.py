"""ctypes binding of ``libmonarch_attn.so`` (argument marshalling only).

Every function here forwards torch tensors' device pointers, their sizes and
the current HIP stream to the C entry point of the same name; all computation
happens in the library's HIP kernels. torch only owns device memory and
streams. The library must have been built (``build.py``); if it is missing,
the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmonarch_attn.so")

MA_OK = 0
MA_BF16 = 0
MA_F32 = 1

_lock = threading.Lock()
_lib = None

_I32 = ctypes.c_int32
_PTR = ctypes.c_void_p
_SIZE = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/monarch_attn.h
SIGNATURES = {
    "ma_workspace_bytes": (_SIZE, [_I32] * 10),
    "monarch_attn_fwd": (ctypes.c_int, [_PTR] * 5 + [_SIZE] + [_I32] * 8 + [_PTR]),
    "monarch_attn_fwd_noalloc": (ctypes.c_int, [_PTR] * 4 + [_I32] * 8 + [_PTR]),
    "ma_noalloc_scratch_bytes": (_SIZE, []),
    "monarch_attn_tiled_fwd": (ctypes.c_int, [_PTR] * 5 + [_SIZE] + [_I32] * 9 + [_PTR]),
    "monarch_attn_causal_fwd": (ctypes.c_int, [_PTR] * 5 + [_SIZE] + [_I32] * 9 + [_PTR]),
    "monarch_attn_chunk_fwd": (ctypes.c_int, [_PTR] * 5 + [_I32] * 10 + [_PTR]),
    "dense_attn_fwd": (ctypes.c_int, [_PTR] * 4 + [_I32] * 5 + [_PTR]),
    "ma_stage_r_fwd": (ctypes.c_int, [_PTR] * 4 + [_I32] * 8 + [_PTR]),
    "ma_stage_l_fwd": (ctypes.c_int, [_PTR] * 4 + [_I32] * 10 + [_PTR]),
    "ma_bwd_workspace_bytes": (_SIZE, [_I32] * 10),
    "monarch_attn_bwd": (ctypes.c_int, [_PTR] * 10 + [_SIZE] + [_I32] * 10 + [_PTR]),
    "ma_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ma_last_hip_error": (ctypes.c_int, []),
}


class MonarchAttnError(RuntimeError):
    def __init__(self, status: int, lib):
        self.status = status
        msg = lib.ma_status_string(status).decode()
        if status == -5:
            msg += " (hipError %d)" % lib.ma_last_hip_error()
        super().__init__(msg)


def load_library(path: Optional[str] = None):
    """Load the shared library (once) and declare every exported signature."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                "HIP library %s is not built; run `python -m structured_attention_video_attn_amd.build`" % p)
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MA_BF16
    if t.dtype == torch.float32:
        return MA_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


def _stream_ptr(t, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _check(*ts):
    """Same dtype, same device, contiguous [batch, heads, N, head_dim] tensors."""
    ref = ts[0]
    for t in ts:
        if t.dim() != 4:
            raise ValueError("tensors must be [batch, heads, N, head_dim]")
        if t.dtype != ref.dtype or t.shape != ref.shape or t.device != ref.device:
            raise ValueError("q, k, v and out must share dtype, shape and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _check_grid(q, T, H, W):
    """The library sees only the grid, never the tensors' size: a grid with more
    tokens than the tensors hold would make the kernels read and write past them."""
    if q.dim() != 4 or min(T, H, W) < 0 or q.shape[2] != T * H * W:
        raise ValueError("q.shape[2] (%s) must equal T*H*W = %d*%d*%d"
                         % (q.shape[2] if q.dim() == 4 else "?", T, H, W))


def _check_workspace(ws, q):
    """A workspace (or cache) buffer: contiguous and on q's GPU (its pointer goes to the kernels)."""
    if ws is None:
        return
    if not ws.is_cuda or ws.device != q.device:
        raise ValueError("workspace must be a GPU tensor on q's device (%s), got %s" % (q.device, ws.device))
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(name, *args):
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != MA_OK:
        raise MonarchAttnError(st, lib)


def ma_workspace_bytes(batch, heads, T, H, W, r_axes=1, tile_t=0, tile_h=0, head_dim=128,
                       dtype=MA_BF16) -> int:
    return int(load_library().ma_workspace_bytes(batch, heads, T, H, W, r_axes, tile_t, tile_h,
                                                 head_dim, dtype))


def monarch_attn_fwd(q, k, v, out, workspace, T, H, W, r_axes=1, stream=None):
    _check_grid(q, T, H, W)
    _check(q, k, v, out)
    _check_workspace(workspace, q)
    B, h, N, d = q.shape
    ws_bytes = _ws_bytes(workspace)
    _call("monarch_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace), ws_bytes,
          B, h, T, H, W, r_axes, d, _dtype_code(q), _stream_ptr(q, stream))
    return out


def monarch_attn_fwd_noalloc(q, k, v, out, T, H, W, r_axes=1, stream=None):
    """monarch_attn_fwd with Y in the library's fixed per-GPU buffer: no workspace, no allocation."""
    _check_grid(q, T, H, W)
    _check(q, k, v, out)
    B, h, N, d = q.shape
    _call("monarch_attn_fwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h, T, H, W, r_axes, d,
          _dtype_code(q), _stream_ptr(q, stream))
    return out


def ma_noalloc_scratch_bytes() -> int:
    return int(load_library().ma_noalloc_scratch_bytes())


def monarch_attn_tiled_fwd(q, k, v, out, workspace, T, H, W, tile_t, tile_h, stream=None):
    _check_grid(q, T, H, W)
    _check(q, k, v, out)
    _check_workspace(workspace, q)
    B, h, N, d = q.shape
    ws_bytes = _ws_bytes(workspace)
    _call("monarch_attn_tiled_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
          ws_bytes, B, h, T, H, W, tile_t, tile_h, d, _dtype_code(q), _stream_ptr(q, stream))
    return out


def monarch_attn_causal_fwd(q, k, v, out, workspace, T, H, W, chunk_t, r_axes=1, stream=None):
    """Chunk-causal Monarch over the whole sequence (bf16): chunks of chunk_t frames."""
    _check_grid(q, T, H, W)
    _check(q, k, v, out)
    _check_workspace(workspace, q)
    B, h, N, d = q.shape
    ws_bytes = _ws_bytes(workspace)
    _call("monarch_attn_causal_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace), ws_bytes,
          B, h, T, H, W, r_axes, chunk_t, d, _dtype_code(q), _stream_ptr(q, stream))
    return out


def monarch_attn_chunk_fwd(q, k, v, y, out, T, H, W, t0, chunk_t, r_axes=1, stream=None):
    """One step with a cache (bf16): frames [t0, t0 + chunk_t) of y and out are written."""
    _check_grid(q, T, H, W)
    if y is None:
        _check(q, k, v, out)
    else:
        _check(q, k, v, out, y)
    B, h, N, d = q.shape
    _call("monarch_attn_chunk_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(out), B, h, T, H, W, r_axes,
          t0, chunk_t, d, _dtype_code(q), _stream_ptr(q, stream))
    return out


def dense_attn_fwd(q, k, v, out, stream=None):
    _check(q, k, v, out)
    B, h, N, d = q.shape
    _call("dense_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h, N, d, _dtype_code(q),
          _stream_ptr(q, stream))
    return out


def ma_stage_r_fwd(q, k, v, y, T, H, W, r_axes=1, stream=None):
    _check_grid(q, T, H, W)
    _check(q, k, v, y)
    B, h, N, d = q.shape
    _call("ma_stage_r_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(y), B, h, T, H, W, r_axes, d,
          _dtype_code(q), _stream_ptr(q, stream))
    return y


def ma_stage_l_fwd(q, k, y, out, T, H, W, r_axes=1, tile_t=0, tile_h=0, stream=None):
    _check_grid(q, T, H, W)
    _check(q, k, y, out)
    B, h, N, d = q.shape
    _call("ma_stage_l_fwd", _ptr(q), _ptr(k), _ptr(y), _ptr(out), B, h, T, H, W, r_axes, tile_t,
          tile_h, d, _dtype_code(q), _stream_ptr(q, stream))
    return out


def ma_bwd_workspace_bytes(batch, heads, T, H, W, r_axes=1, tile_t=0, tile_h=0, head_dim=128,
                           dtype=MA_BF16) -> int:
    return int(load_library().ma_bwd_workspace_bytes(batch, heads, T, H, W, r_axes, tile_t, tile_h,
                                                     head_dim, dtype))


def monarch_attn_bwd(q, k, v, out, dout, dq, dk, dv, workspace, T, H, W, r_axes=1, tile_t=0,
                     tile_h=0, stream=None, y=None):
    """dq, dk, dv of the forward (same r_axes / tile) given dout; bf16 only. `y`: the
    forward's Y (its workspace viewed as q's shape) to skip recomputing stage R, or None."""
    _check_grid(q, T, H, W)
    _check(q, k, v, out, dout, dq, dk, dv)
    if y is not None:
        _check(q, y)
    _check_workspace(workspace, q)
    B, h, N, d = q.shape
    ws_bytes = _ws_bytes(workspace)
    _call("monarch_attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(y), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, h, T, H, W, r_axes, tile_t, tile_h, d,
          _dtype_code(q), _stream_ptr(q, stream))
    return dq, dk, dv
