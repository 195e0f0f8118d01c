"""Build the gfx950 HIP library libmoe_mi355x.so in-tree with hipcc.

    python -m mixture_experts_layer_24_amd.build      (or build() from Python)

Every .hip file under csrc/ is compiled for gfx950 and linked into one shared
library next to this file.  Packed-FP32 instruction selection is switched
off for the device code (hipcc's host pass warns that it does not know that
target feature; the warning is harmless).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources()]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
