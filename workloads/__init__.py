"""Seeded synthetic Q/K/V for the video-attention workloads.

This module only draws inputs. It holds no attention arithmetic, and both the
HIP path (through the tests and the bench) and the CPU oracle consume what it
returns. Arrays come back as float32 NumPy arrays shaped ``[batch, heads, N, d]``
with token ``n = (t*H + h)*W + w`` (w fastest), the flattening of a
``(T, H, W)`` video token grid.

Workloads (grid, heads, head_dim, storage dtype, value recipe):

* ``tiny``       2x4x4 grid,   1 head,  d16,  fp32, Q/K/V ~ N(0,1)
* ``chunk``      3x30x52,      12 heads, d128, bf16, Q,K ~ N(0,1)/d^0.25, V ~ N(0,1)
* ``full``       21x30x52,     12 heads, d128, bf16, same recipe as ``chunk``
* ``structured`` 21x30x52,     12 heads, d128, bf16, periodic positional
  features + N(0, 0.1^2) noise + 2% planted long-range pairs; tile 3 frames x 30 rows
* ``long``       81x30x52,     16 heads, d128, bf16, Q/K/V ~ N(0,1); tile 9 frames x 30 rows
* ``chunk_sharp`` / ``full_sharp``: the ``chunk``/``full`` shapes with unscaled
  N(0,1) Q/K (logit std 1), so that the softmax is far from flat.

The 30x52 per-frame grid stands in for the 480p latent grid of the video
models the MonarchRT pages evaluate on; the pages never print their token grid.

The chunk-causal (autoregressive) workload uses the ``full`` inputs with chunks
of ``CAUSAL_CHUNK_T`` frames: the ``chunk`` shape (3 frames) is one generation
step's query chunk, and the step with a cache is the last chunk, frames 18..20,
attending to all 21 frames.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "CAUSAL_CHUNK_T", "make_qkv", "to_bf16_f32"]

CAUSAL_CHUNK_T = 3   # frames per autoregressive chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    batch: int
    heads: int
    head_dim: int
    dtype: str              # "bf16" or "f32": storage/compute-input type
    recipe: str             # "normal", "scaled_qk" or "structured"
    seed: int
    tile: Optional[Tuple[int, int]] = None   # (tile_t, tile_h) for the tiled variant

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.n_tokens, self.head_dim)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 4, 4, 1, 1, 16, "f32", "normal", 0, (1, 2)),
    "chunk": Workload("chunk", 3, 30, 52, 1, 12, 128, "bf16", "scaled_qk", 1, (3, 30)),
    "full": Workload("full", 21, 30, 52, 1, 12, 128, "bf16", "scaled_qk", 2, (3, 30)),
    "structured": Workload("structured", 21, 30, 52, 1, 12, 128, "bf16", "structured", 3, (3, 30)),
    "long": Workload("long", 81, 30, 52, 1, 16, 128, "bf16", "normal", 4, (9, 30)),
    "chunk_sharp": Workload("chunk_sharp", 3, 30, 52, 1, 12, 128, "bf16", "normal", 11, (3, 30)),
    "full_sharp": Workload("full_sharp", 21, 30, 52, 1, 12, 128, "bf16", "normal", 12, (3, 30)),
}

# Constants of the structured recipe (chosen here, not taken from the pages):
# 21 harmonics per grid axis, feature gain so that a token's zero-displacement
# logit is 4, noise std 0.1, 2% planted pairs whose boost adds 6 to their logit,
# partners at least 7 frames apart.
_HARMONICS = 21
_POS_LOGIT = 4.0
_NOISE_STD = 0.1
_PLANT_FRACTION = 0.02
_PLANT_LOGIT = 6.0
_PLANT_MIN_DT = 7


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Pure bit manipulation, identical to what torch's float32->bfloat16 cast does
    for finite values; used so that tests can hand the same rounded values to
    the GPU (as bf16) and to the oracle (as float64).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = 0x7FFF + ((u >> 16) & 1)
    r = ((u + rounding) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def _positional_features(T: int, H: int, W: int, d: int) -> np.ndarray:
    """Periodic, axis-separable features phi(t,h,w), shape [T*H*W, d]."""
    feats = []
    for axis_len, axis in ((T, 0), (H, 1), (W, 2)):
        coord = np.indices((T, H, W))[axis].reshape(-1).astype(np.float64)
        for kk in range(1, _HARMONICS + 1):
            ang = 2.0 * math.pi * kk * coord / axis_len
            feats.append(np.cos(ang))
            feats.append(np.sin(ang))
    phi = np.stack(feats, axis=1)
    if phi.shape[1] > d:
        raise ValueError("structured recipe needs head_dim >= %d" % phi.shape[1])
    out = np.zeros((phi.shape[0], d), dtype=np.float64)
    out[:, : phi.shape[1]] = phi
    return out


def _structured_head(rng: np.random.Generator, wl: Workload, phi: np.ndarray):
    n, d = phi.shape
    scale = 1.0 / math.sqrt(d)
    n_feat = 3 * _HARMONICS
    alpha = math.sqrt(_POS_LOGIT / (n_feat * scale))
    beta = math.sqrt(_PLANT_LOGIT / scale)
    q = alpha * phi + _NOISE_STD * rng.standard_normal((n, d))
    k = alpha * phi + _NOISE_STD * rng.standard_normal((n, d))
    n_plant = int(round(_PLANT_FRACTION * n))
    queries = rng.choice(n, size=n_plant, replace=False)
    t_of = np.arange(n) // (wl.H * wl.W)
    for qi in queries:
        far = np.nonzero(np.abs(t_of - t_of[qi]) >= _PLANT_MIN_DT)[0]
        kj = far[rng.integers(0, far.size)] if far.size else qi
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        q[qi] += beta * u
        k[kj] += beta * u
    v = rng.standard_normal((n, d))
    return q, k, v


def make_qkv(wl: Workload, heads: Optional[int] = None, seed: Optional[int] = None,
             round_bf16: Optional[bool] = None):
    """Draw (q, k, v) for a workload, float32 arrays of shape [batch, heads, N, d].

    ``heads`` overrides the head count (a prefix of the same stream is NOT
    guaranteed; each call draws afresh from ``seed``). When the workload's
    dtype is bf16 (or ``round_bf16`` is set) the values are rounded to bf16.

    Draw order: NumPy PCG64 ``default_rng(seed)``; for the "normal" and
    "scaled_qk" recipes q, k, v are drawn in that order with
    ``standard_normal(shape, float32)``; "scaled_qk" then divides q and k by
    d**0.25. The "structured" recipe draws per (batch, head): q-noise, k-noise,
    planted query set, then per planted query its partner and unit vector, then v.
    """
    h = wl.heads if heads is None else heads
    s = wl.seed if seed is None else seed
    rng = np.random.default_rng(s)
    shape = (wl.batch, h, wl.n_tokens, wl.head_dim)
    if wl.recipe in ("normal", "scaled_qk"):
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if wl.recipe == "scaled_qk":
            f = np.float32(wl.head_dim ** -0.25)
            q *= f
            k *= f
    elif wl.recipe == "structured":
        phi = _positional_features(wl.T, wl.H, wl.W, wl.head_dim)
        q = np.empty(shape, np.float32)
        k = np.empty(shape, np.float32)
        v = np.empty(shape, np.float32)
        for b in range(wl.batch):
            for hh in range(h):
                qh, kh, vh = _structured_head(rng, wl, phi)
                q[b, hh], k[b, hh], v[b, hh] = qh, kh, vh
    else:
        raise ValueError("unknown recipe " + wl.recipe)
    rb = (wl.dtype == "bf16") if round_bf16 is None else round_bf16
    if rb:
        q, k, v = to_bf16_f32(q), to_bf16_f32(k), to_bf16_f32(v)
    return q, k, v
