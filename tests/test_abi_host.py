"""CPU tests of the C ABI: symbols, argument checks, error codes and group addressing.

Nothing here launches a kernel. Every call below either fails an argument
check (which the library performs before any HIP call) or describes an empty
problem; the group addressing is exercised through a host-only build of the
library's own headers (tests/host/group_enum.cpp).
"""
import ctypes
import os
import re
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "monarch_attn.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, -1, -2, -3, -4
BF16, F32 = 0, 1


@pytest.fixture(scope="module")
def lib():
    from structured_attention_video_attn_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from structured_attention_video_attn_amd import build
        build.build()
    return _binding.load_library()


@pytest.fixture(scope="module")
def group_enum(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("host") / "group_enum")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-o", exe,
                    os.path.join(ROOT, "tests", "host", "group_enum.cpp")], check=True)
    return exe


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_symbols_exported(lib):
    names = header_functions()
    assert set(names) >= {"monarch_attn_fwd", "monarch_attn_tiled_fwd", "dense_attn_fwd",
                          "ma_workspace_bytes", "ma_status_string", "ma_stage_r_fwd",
                          "ma_stage_l_fwd", "ma_last_hip_error"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, 17):
        s = lib.ma_status_string(st)
        assert s is not None and len(s) > 0
    assert lib.ma_status_string(-4).startswith(b"MA_ERR_WORKSPACE")
    assert lib.ma_last_hip_error() == 0


def test_workspace_bytes(lib):
    ws = lib.ma_workspace_bytes
    assert ws(1, 12, 21, 30, 52, 1, 0, 0, 128, BF16) == 12 * 32760 * 128 * 2
    assert ws(2, 3, 2, 4, 4, 1, 0, 0, 16, F32) == 2 * 3 * 32 * 16 * 4
    assert ws(1, 12, 21, 30, 52, 1, 3, 30, 128, BF16) == 12 * 32760 * 128 * 2
    assert ws(1, 1, 2, 4, 4, 3, 0, 0, 16, F32) == 0      # one block: Y goes straight to out
    assert ws(1, 1, 2, 4, 4, 0, 0, 0, 16, F32) == 0      # b2 = 1: stage L reads V
    assert ws(1, 1, 2, 4, 4, 1, 1, 1, 16, F32) == 0      # 1x1 tiles: stage L is the identity
    assert ws(1, 1, 2, 4, 4, 1, 0, 0, 48, F32) == 0      # unsupported head_dim
    assert ws(0, 1, 2, 4, 4, 1, 0, 0, 16, F32) == 0      # empty


A16 = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
BIG = 1 << 30


def _ptrs(n=5, stride=BIG):
    return [A16 + i * stride for i in range(n)]


def test_monarch_argument_errors(lib):
    f = lib.monarch_attn_fwd
    q, k, v, o, w = _ptrs()
    nb = 12 * 32760 * 128 * 2
    good = dict(batch=1, heads=12, T=21, H=30, W=52, r=1, d=128, dt=BF16)

    def call(q=q, k=k, v=v, o=o, w=w, wb=nb, **kw):
        a = dict(good, **kw)
        return f(q, k, v, o, w, wb, a["batch"], a["heads"], a["T"], a["H"], a["W"], a["r"], a["d"],
                 a["dt"], None)

    assert call(q=None) == INVALID
    assert call(o=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(heads=-3) == INVALID
    assert call(r=4) == INVALID
    assert call(r=-1) == INVALID
    assert call(d=48) == UNSUPPORTED
    assert call(d=256) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(q=A16 + 8) == ALIGN
    assert call(o=A16 + 4 * BIG + 2) == ALIGN
    assert call(w=None) == WORKSPACE
    assert call(wb=nb - 1) == WORKSPACE
    assert call(w=A16 + 4 * BIG + 8) == ALIGN
    assert call(o=q) == INVALID                     # out aliases q
    assert call(o=k + 4096) == INVALID              # out overlaps k
    assert call(w=v) == INVALID                     # workspace aliases v
    assert call(w=o + 2 * 16) == INVALID            # workspace overlaps out
    assert call(T=1 << 20, H=1 << 10, W=1) == UNSUPPORTED   # N*d beyond 32-bit offsets
    # empty problems are no-ops, even with null pointers
    assert call(q=None, k=None, v=None, o=None, w=None, batch=0) == OK
    assert call(q=None, k=None, v=None, o=None, w=None, W=0) == OK


def test_noalloc_argument_errors(lib):
    # Every check of the no-allocation entry point runs before any HIP call,
    # including the size limit of its fixed per-GPU buffer.
    SCRATCH = -6
    f = lib.monarch_attn_fwd_noalloc
    cap = lib.ma_noalloc_scratch_bytes()
    assert cap == 128 << 20
    q, k, v, o = _ptrs(4)

    def call(q=q, k=k, v=v, o=o, batch=1, heads=12, T=21, H=30, W=52, r=1, d=128, dt=BF16):
        return f(q, k, v, o, batch, heads, T, H, W, r, d, dt, None)

    assert lib.ma_workspace_bytes(1, 24, 21, 30, 52, 1, 0, 0, 128, BF16) > cap
    assert call(heads=24) == SCRATCH               # Y of 201 MB does not fit
    assert call(heads=12, dt=F32) == SCRATCH       # fp32: Y of 201 MB
    assert call(q=None) == INVALID
    assert call(o=q) == INVALID
    assert call(v=A16 + 2 * BIG + 8) == ALIGN
    assert call(r=5) == INVALID
    assert call(d=24) == UNSUPPORTED
    assert call(q=None, k=None, v=None, o=None, heads=0) == OK
    assert lib.ma_status_string(SCRATCH).startswith(b"MA_ERR_SCRATCH")


def test_tiled_and_stage_argument_errors(lib):
    q, k, v, o, w = _ptrs()
    nb = 1 << 28
    t = lib.monarch_attn_tiled_fwd
    assert t(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 0, 30, 128, BF16, None) == INVALID
    assert t(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 3, -1, 128, BF16, None) == INVALID
    assert t(q, k, v, o, None, 0, 1, 12, 21, 30, 52, 3, 30, 128, BF16, None) == WORKSPACE
    assert t(q, k, v, q, w, nb, 1, 12, 21, 30, 52, 3, 30, 128, BF16, None) == INVALID
    assert t(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 3, 30, 24, BF16, None) == UNSUPPORTED
    assert t(None, None, None, None, None, 0, 1, 0, 21, 30, 52, 3, 30, 128, BF16, None) == OK
    r = lib.ma_stage_r_fwd
    assert r(q, k, v, q, 1, 12, 21, 30, 52, 1, 128, BF16, None) == INVALID
    assert r(q, k, v, o, 1, 12, 21, 30, 52, 7, 128, BF16, None) == INVALID
    assert r(q, k, v, o + 8, 1, 12, 21, 30, 52, 1, 128, BF16, None) == ALIGN
    l = lib.ma_stage_l_fwd
    assert l(q, k, v, o, 1, 12, 21, 30, 52, 2, 3, 30, 128, BF16, None) == INVALID  # tiles need r_axes 1
    assert l(q, k, v, o, 1, 12, 21, 30, 52, 1, 3, 0, 128, BF16, None) == INVALID
    assert l(q, k, o, o, 1, 12, 21, 30, 52, 1, 0, 0, 128, BF16, None) == INVALID   # out aliases y
    d = lib.dense_attn_fwd
    assert d(q, k, v, None, 1, 12, 4680, 128, BF16, None) == INVALID
    assert d(q, k, v, o, 1, 12, -5, 128, BF16, None) == INVALID
    assert d(q, k, v, o, 1, 12, 4680, 100, BF16, None) == UNSUPPORTED
    assert d(q, k, v, v, 1, 12, 4680, 128, BF16, None) == INVALID
    assert d(None, None, None, None, 1, 12, 0, 128, BF16, None) == OK


def test_backward_workspace_and_argument_errors(lib):
    wsb = lib.ma_bwd_workspace_bytes
    tb = 12 * 32760 * 128 * 2
    # Y, dY, then (lse, D) per member: stage L groups of 630 (stride 768), stage R groups of 52 (stride 192)
    stats_l = 12 * 52 * 768 * 8
    stats_r = 12 * 630 * 192 * 8
    r256 = lambda x: (x + 255) // 256 * 256
    assert wsb(1, 12, 21, 30, 52, 1, 0, 0, 128, BF16) == 2 * r256(tb) + r256(stats_l) + r256(stats_r)
    assert wsb(1, 12, 21, 30, 52, 1, 0, 0, 128, F32) == 0      # backward is bf16 only
    assert wsb(1, 12, 21, 30, 52, 1, 0, 0, 48, BF16) == 0      # unsupported head_dim
    assert wsb(0, 12, 21, 30, 52, 1, 0, 0, 128, BF16) == 0     # empty
    f = lib.monarch_attn_bwd
    q, k, v, o, do, dq, dk, dv, w, y = _ptrs(10)
    nb = wsb(1, 12, 21, 30, 52, 1, 0, 0, 128, BF16)

    def call(q=q, k=k, v=v, o=o, do=do, y=None, dq=dq, dk=dk, dv=dv, w=w, wb=nb, r=1, tt=0, th=0, d=128,
             dt=BF16, batch=1):
        return f(q, k, v, o, do, y, dq, dk, dv, w, wb, batch, 12, 21, 30, 52, r, tt, th, d, dt, None)

    assert call(dt=F32) == UNSUPPORTED
    assert call(d=48) == UNSUPPORTED
    assert call(do=None) == INVALID
    assert call(dv=None) == INVALID
    assert call(dk=A16 + 6 * BIG + 4) == ALIGN
    assert call(dq=q) == INVALID                    # a gradient aliases an input
    assert call(dv=dk) == INVALID                   # two gradients alias
    assert call(w=None) == WORKSPACE
    assert call(wb=nb - 1) == WORKSPACE
    assert call(w=do) == INVALID                    # workspace aliases dout
    assert call(w=do + 4096) == INVALID             # workspace starts inside dout
    assert call(w=A16 + 9 * BIG, k=A16 + 9 * BIG + nb - 16) == INVALID   # k starts inside the workspace
    assert call(r=2, tt=3, th=30) == INVALID        # tiles need r_axes 1
    assert call(y=y + 4) == ALIGN                   # the forward's Y, misaligned
    assert call(y=w + 4096) == INVALID              # ... inside the workspace
    assert call(y=dk) == INVALID                    # ... aliasing a gradient
    assert call(y=y + 4, dt=F32) == UNSUPPORTED     # dtype is checked first
    assert call(q=None, k=None, v=None, o=None, do=None, dq=None, dk=None, dv=None, w=None, batch=0) == OK


def _parse_groups(text):
    r, l = [], []
    lines = text.strip().splitlines()
    trivial = tuple(int(x) for x in lines[0].split()[1:])
    for line in lines[1:]:
        tag, rest = line.split(" ", 1)
        toks = [int(x) for x in rest.split(":")[1].split()]
        (r if tag == "R" else l).append(frozenset(toks))
    return trivial, r, l


GRIDS = [
    ((2, 4, 4), 1, None), ((2, 4, 4), 2, None), ((2, 4, 4), 3, None), ((2, 4, 4), 0, None),
    ((3, 5, 7), 1, None), ((3, 5, 7), 1, (2, 2)), ((3, 5, 7), 1, (1, 5)), ((3, 5, 7), 1, (3, 1)),
    ((3, 5, 7), 1, (4, 9)), ((4, 3, 2), 1, (3, 2)), ((2, 4, 4), 1, (1, 2)), ((7, 6, 5), 1, (3, 4)),
    ((3, 30, 52), 1, None), ((21, 30, 52), 1, (3, 30)), ((5, 7, 3), 2, None),
]


@pytest.mark.parametrize("grid,r_axes,tile", GRIDS)
def test_group_addressing_matches_oracle(group_enum, grid, r_axes, tile):
    T, H, W = grid
    tt, th = tile if tile else (0, 0)
    out = subprocess.run([group_enum, "groups", str(T), str(H), str(W), str(r_axes), str(tt), str(th)],
                         capture_output=True, text=True, check=True).stdout
    (r_triv, l_triv), r_groups, l_groups = _parse_groups(out)
    want_r = [frozenset(g.tolist()) for g in oracle.stage_r_groups(grid, r_axes)]
    want_l = [frozenset(g.tolist()) for g in oracle.stage_l_groups(grid, r_axes, tile)]
    assert sorted(map(sorted, r_groups)) == sorted(map(sorted, want_r))
    assert sorted(map(sorted, l_groups)) == sorted(map(sorted, want_l))
    assert r_triv == int(all(len(g) == 1 for g in want_r))
    assert l_triv == int(all(len(g) == 1 for g in want_l))


def test_xcd_remap_is_bijective(group_enum):
    out = subprocess.run([group_enum, "remap", "4100"], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "ok"


def test_binding_fails_loudly_without_library(tmp_path):
    from structured_attention_video_attn_amd import _binding
    with pytest.raises(RuntimeError, match="not built"):
        _binding.load_library(str(tmp_path / "missing.so"))


def test_causal_and_chunk_argument_errors(lib):
    # every call fails an argument check or is empty: nothing is launched
    q, k, v, o, w = _ptrs()
    nb = 12 * 32760 * 128 * 2
    c = lib.monarch_attn_causal_fwd
    assert c(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 1, 0, 128, BF16, None) == INVALID     # chunk_t < 1
    assert c(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 3, 3, 128, BF16, None) == INVALID     # r_axes 3
    assert c(q, k, v, o, w, nb, 1, 12, 21, 30, 52, 1, 3, 128, F32, None) == UNSUPPORTED
    assert c(q, k, v, q, w, nb, 1, 12, 21, 30, 52, 1, 3, 128, BF16, None) == INVALID     # out aliases q
    assert c(q, k, v, o, None, 0, 1, 12, 21, 30, 52, 1, 3, 128, BF16, None) == WORKSPACE
    assert c(None, None, None, None, None, 0, 0, 12, 21, 30, 52, 1, 3, 128, BF16, None) == OK
    s = lib.monarch_attn_chunk_fwd
    y = w
    good = (1, 12, 21, 30, 52)
    assert s(q, k, v, y, o, *good, 3, 18, 3, 128, BF16, None) == INVALID       # r_axes 3
    assert s(q, k, v, y, o, *good, 1, -1, 3, 128, BF16, None) == INVALID      # t0 < 0
    assert s(q, k, v, y, o, *good, 1, 19, 3, 128, BF16, None) == INVALID      # past the last frame
    assert s(q, k, v, y, o, *good, 1, 18, 0, 128, BF16, None) == INVALID      # chunk_t < 1
    assert s(q, k, v, y, o, *good, 1, 18, 3, 128, F32, None) == UNSUPPORTED
    assert s(q, k, v, None, o, *good, 1, 18, 3, 128, BF16, None) == INVALID   # y needed at r_axes 1
    assert s(q, k, v, o, o, *good, 1, 18, 3, 128, BF16, None) == INVALID     # y aliases out
    assert s(q, k, v, v, o, *good, 1, 18, 3, 128, BF16, None) == INVALID     # y aliases v
    assert s(q, k, v, y + 8, o, *good, 1, 18, 3, 128, BF16, None) == ALIGN
    assert s(q, k, v, y, q, *good, 1, 18, 3, 128, BF16, None) == INVALID     # out aliases q
    assert s(q, k, v, y, o, 1, 12, 21, 30, 52, 1, 18, 3, 48, BF16, None) == UNSUPPORTED
    assert s(None, None, None, None, None, 0, 12, 21, 30, 52, 1, 18, 3, 128, BF16, None) == OK


def test_binding_rejects_grid_that_does_not_match_tensors():
    # The C ABI never sees the tensors' token count: the binding must refuse a grid
    # whose T*H*W differs from q.shape[2] before any pointer reaches the library.
    import torch
    import structured_attention_video_attn_amd as ma
    q = torch.empty(1, 2, 30, 16)
    calls = [
        lambda: ma.monarch_attn_fwd(q, q, q, q, None, 2, 4, 4),
        lambda: ma.monarch_attn_tiled_fwd(q, q, q, q, None, 2, 4, 4, 1, 2),
        lambda: ma.monarch_attn_causal_fwd(q, q, q, q, None, 2, 4, 4, 1),
        lambda: ma.monarch_attn_chunk_fwd(q, q, q, q, q, 2, 4, 4, 0, 1),
        lambda: ma.ma_stage_r_fwd(q, q, q, q, 2, 4, 4),
        lambda: ma.ma_stage_l_fwd(q, q, q, q, 2, 4, 4),
        lambda: ma.monarch_attn_bwd(q, q, q, q, q, q, q, q, None, 2, 4, 4),
    ]
    for call in calls:
        with pytest.raises(ValueError, match=r"T\*H\*W"):
            call()


def test_binding_rejects_host_workspace():
    import torch
    from structured_attention_video_attn_amd import _binding
    q = torch.empty(1, 1, 32, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding._check_workspace(torch.empty(512), q)
    _binding._check_workspace(None, q)   # no workspace: nothing to check
