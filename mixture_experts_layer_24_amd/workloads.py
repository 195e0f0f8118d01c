"""The five MoE-layer workloads, as plain data (no arithmetic of the method).

Shapes follow the pages' model family (the 350M+MoE-128 and 1.3B+MoE-128
models of "DeepSpeed-MoE: Advancing Mixture-of-Experts Inference and
Training ..." notes, sec. 2.1: top-1, 128 experts on every other FFN; its
sec. 3.1 Residual-MoE for the PR-MoE layer), a decode regime (one token per
sequence, "DeepSpeed MoE and Model Compression", section "MoE Inference")
and a skewed top-2 layer with symmetric int8 expert weights (the survey
notes, sec. 1.2.2 and 1.2.3.1 weight-only quantisation).

Fields:
  T, d, E, k, d_ff     tokens, model dim, experts, top-k, expert hidden dim
  d_ff_dense           width of PR-MoE's fixed dense MLP (0 = no PR-MoE)
  capacity_factor      C = min(T, ceil(k*T*cf/E))
  act                  'f32' | 'bf16'  (x, router and plain weights, outputs)
  wfmt                 'plain' | 'int8'  (expert weights; int8 uses fp16
                       scales per 128 input-dim elements of each output row)
  pr_moe, add_skip     y = [x] + [dense MLP(x)] + sum_j g_j Expert_j(x)
  zipf_s               router bias b_e = -s*ln(e+1) (0 = no bias)
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    capacity_factor: float
    act: str = "bf16"
    wfmt: str = "plain"
    d_ff_dense: int = 0
    pr_moe: bool = False
    add_skip: bool = True
    normalize_topk: bool = True
    zipf_s: float = 0.0
    x_std: float = 1.0
    w_std: float = 0.02
    aux_alpha: float = 1.0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny fp32 layer: drops on (capacity 16 for 64 tokens over 4 experts)
    "tiny_f32": Workload("tiny_f32", T=64, d=32, E=4, k=1, d_ff=64,
                         capacity_factor=1.0, act="f32"),
    # 350M+MoE-128 layer shape, 4 sequences x 2048 tokens flattened batch-major
    "moe128_350m": Workload("moe128_350m", T=8192, d=1024, E=128, k=1,
                            d_ff=4096, capacity_factor=1.0),
    # 1.3B+PR-MoE-128 layer: fixed dense MLP plus one top-1 residual expert,
    # y = MLP(x) + g * Expert(x)
    "prmoe128_1p3b": Workload("prmoe128_1p3b", T=16384, d=2048, E=128, k=1,
                              d_ff=8192, capacity_factor=1.0, d_ff_dense=8192,
                              pr_moe=True, add_skip=False),
    # decode: one token per sequence, top-2 renormalised, no drops (cf = E/k)
    "decode_top2": Workload("decode_top2", T=32, d=4096, E=64, k=2, d_ff=14336,
                            capacity_factor=32.0),
    # skewed top-2 with int8 experts; Zipf(1.2) router prior forces drops
    "skewed_top2_int8": Workload("skewed_top2_int8", T=32768, d=4096, E=64, k=2,
                                 d_ff=14336, capacity_factor=1.25, wfmt="int8",
                                 zipf_s=1.2),
}

# the workload the headline metric (1.3B+MoE-128 shape) is quoted on
HEADLINE = "prmoe128_1p3b"
