"""Build libbeam_moe.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbeam_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions are kept out of every kernel on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False, extra=None, out: str = LIB) -> str:
    cmd = [HIPCC] + FLAGS + list(extra or []) + ["-I", os.path.join(ROOT, "include")] + sources() + ["-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libbeam_moe build failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    if verbose:
        print(" ".join(cmd))
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if msg.strip():
            print(msg)
    return out


if __name__ == "__main__":
    build(verbose=True)
