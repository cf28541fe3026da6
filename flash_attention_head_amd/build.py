"""Build step of the HIP library (``libsdpa_mi355x.so``, in-tree, gfx950 only).

Run as ``python -m flash_attention_head_amd.build``; ``__graft_entry__.build()``
calls :func:`build` too.  hipcc cross-compiles for gfx950 without a GPU.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsdpa_mi355x.so")
SOURCES = [os.path.join(PKG, "csrc", "attn_kernels.hip"), os.path.join(PKG, "csrc", "sdpa_api.cpp"),
           os.path.join(PKG, "csrc", "sdpa_noalloc.hip"), os.path.join(PKG, "csrc", "attn_q4_decode.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax rescale and the epilogue
    # read them with VALU instructions, and AGPR accumulators made the register
    # allocator copy the whole output tile between register files every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = LIB, extra: tuple = ()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
