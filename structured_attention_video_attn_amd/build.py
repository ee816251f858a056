"""Build the HIP library in-tree: ``libmonarch_attn.so`` for gfx950.

Run ``python -m structured_attention_video_attn_amd.build`` (or call ``build()``).
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmonarch_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, "monarch_attn.hip")]
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags():
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fno-strict-aliasing",
        # no kernel relies on NaN semantics (masked scores are -inf): lets fmaxf
        # map to one v_max/v_max3 without canonicalising its MFMA-produced inputs
        "-fno-honor-nans",
        # keep the compiler from forming packed fp32 vector ops (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library; returns its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc_path()] + compile_flags() + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed with exit code %d" % res.returncode)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
