"""Negative and positive controls for the bf16 parity gates (CPU only).

At the flat-logit workloads (Q, K ~ N(0,1)/d^0.25) the softmax of both stages
is nearly uniform, so every output row sits close to the head's mean of V and
a max-abs gate of 2e-2 alone cannot tell a correct kernel from one that ignores
Q and K. The relative gates of parity_util (G1: relative L2 error; G2: error
against the spread of the reference around its mean) carry the check there.
These tests show that they do: with the fp64 oracle's output as reference,

* an all-zero output, the head's global-mean output, and stage L run over the
  wrong stride (token sets n mod (W +- 1) instead of n mod W, i.e. a kernel
  whose gather uses the wrong permutation) each fail G1 or G2;
* the oracle's own output rounded the way the bf16 path rounds (Y and O stored
  in bf16) passes every gate.

The block structure that makes the flat case possible is the aligned split
(b1, b2) = (f*h, w) of the MonarchRT summaries (zh 2.2).
"""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_qkv, to_bf16_f32

from parity_util import G1_MAX, G2_MAX, MAX_ABS_BF16, errors


def _fails_relative_gates(got, ref):
    _, g1, g2 = errors(got, ref)
    return g1 > G1_MAX or g2 > G2_MAX


def _wrong_stride(q, k, y, stride):
    """Stage L over the token sets {n : n mod stride = i} (a wrong permutation)."""
    n = q.shape[2]
    groups = [np.arange(i, n, stride) for i in range(stride)]
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = oracle.group_softmax_attention(q[b, h].astype(np.float64), k[b, h].astype(np.float64),
                                                       y[b, h], groups)
    return out


@pytest.mark.parametrize("name", ["chunk", "full"])
def test_gates_reject_wrong_outputs_and_accept_rounded_oracle(name):
    wl = WORKLOADS[name]
    grid = (wl.T, wl.H, wl.W)
    heads = 12 if name == "chunk" else 3
    q, k, v = make_qkv(wl, heads=heads)
    ref, y = oracle.monarch_attention(q, k, v, grid, return_y=True)

    zeros = np.zeros_like(ref)
    mean = np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), ref.shape)
    controls = {"zeros": zeros, "global mean": mean,
                "stride W+1": _wrong_stride(q, k, y, wl.W + 1),
                "stride W-1": _wrong_stride(q, k, y, wl.W - 1)}
    for label, bad in controls.items():
        assert _fails_relative_gates(bad, ref), "%s %s passes G1 and G2" % (name, label)

    # The weakness the relative gates exist for: at these flat workloads the
    # global-mean output is within the max-abs gate.
    assert errors(mean, ref)[0] <= MAX_ABS_BF16

    # An honest bf16 result: Y rounded to bf16 before stage L, the output rounded to bf16.
    y16 = to_bf16_f32(y.astype(np.float32)).astype(np.float64)
    o16 = oracle.stage_l(q, k, y16, grid)
    o16 = to_bf16_f32(o16.astype(np.float32)).astype(np.float64)
    max_abs, g1, g2 = errors(o16, ref)
    assert max_abs <= MAX_ABS_BF16 and g1 <= G1_MAX and g2 <= G2_MAX, (max_abs, g1, g2)
