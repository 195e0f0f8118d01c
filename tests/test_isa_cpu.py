"""ISA checks of the gfx950 build that need no GPU.

The DMA GEMMs issue global_load_lds_dwordx4 from inline assembly after
setting m0 themselves.  The compiler treats m0 as reserved (it ignores the asm
clobber), so this is only correct while compiler-generated code in those
kernels never reads or writes m0.  Compile gemm.hip and backward.hip to
assembly and check that every m0 access in the DMA kernels is one of the
asm's own "s_mov_b32 m0" writes, each directly followed by its load.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_24_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", [("gemm.hip", "gemm_dma"), ("backward.hip", "gemm_dmag"),
                                        ("backward.hip", "gemm_dwk"),
                                        ("router.hip", "router_dma")])
def test_dma_kernels_use_m0_only_for_their_own_loads(tmp_path, src, kernel):
    out = tmp_path / "k.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S",
                    "--offload-device-only", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I", CSRC, os.path.join(CSRC, src),
                    "-o", str(out)], check=True, capture_output=True)
    asm = out.read_text()
    funcs = re.split(r"\n(?=_Z\S+:)", asm)
    dma = [f for f in funcs if kernel in f.split(":", 1)[0]]
    assert dma, "no DMA kernels found"
    for f in dma:
        lines = [l.strip() for l in f.splitlines() if l.strip() and not l.strip().startswith(";")]
        for i, l in enumerate(lines):
            if re.search(r"\bm0\b", l):
                assert l.startswith("s_mov_b32 m0,"), f"unexpected m0 use: {l}"
                assert lines[i + 1].startswith("global_load_lds_dwordx4"), lines[i + 1]
            assert "movrel" not in l and "gpr_idx" not in l
