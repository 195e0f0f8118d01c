"""Seeded synthetic inputs for the MoE layer.

This module is the one thing the HIP path's tests and the CPU oracle's tests
take from a common place.  It draws random numbers and rounds them to the
storage formats; it contains none of the layer's arithmetic.

Recipe (per workload, see ``workloads.py``):
  x        ~ N(0, x_std^2), drawn in fp32, rounded to the activation format
  W_r      ~ N(0, w_std^2)  [E, d]          (router weights, [out, in])
  b_r      = -zipf_s * ln(e + 1), fp32      (only when zipf_s > 0: a logit
             prior whose softmax alone is a Zipf law over the experts)
  W1[e]    ~ N(0, w_std^2)  [d_ff, d]       one sub-seed per expert
  W2[e]    ~ N(0, w_std^2)  [d, d_ff]
  Wm1, Wm2 ~ N(0, w_std^2)  [d_ff_dense, d], [d, d_ff_dense] (PR-MoE)
  int8 experts: codes uniform on the integers -127..127 and fp16 scales
             uniform in [0.5, 1.5] * w_std / 73.6 (73.6 is the standard
             deviation of that uniform code), one scale per 128 consecutive
             input-dim elements of each output row; with pow2_scales the
             scales are 2^-12 or 2^-13 so every dequantised weight is exactly
             a bfloat16 value.
Rounding to bfloat16 is round-to-nearest-even (torch's ``.to``).

Each tensor (and each expert's weights) has its own sub-seed, so a test can
regenerate any part alone.  Values depend on the device's generator (CPU:
Mersenne twister, GPU: Philox), so a test generates once and copies.
"""
from __future__ import annotations

import math
import zlib

import torch

from .workloads import Workload

CODE_STD = 73.6  # std of the discrete uniform law on -127..127


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(zlib.crc32(f"{seed}/{tag}".encode()) & 0x7FFFFFFF)
    return g


def _act_dtype(wl: Workload):
    return torch.float32 if wl.act == "f32" else torch.bfloat16


def normal(shape, std, seed, tag, device, dtype):
    g = _gen(seed, tag, device)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(dtype)


def int8_codes(shape, seed, tag, device):
    g = _gen(seed, tag, device)
    return torch.randint(-127, 128, shape, generator=g, device=device,
                         dtype=torch.int8)


def fp16_scales(shape, w_std, seed, tag, device, pow2=False):
    g = _gen(seed, tag, device)
    if pow2:
        e = torch.randint(12, 14, shape, generator=g, device=device)
        return torch.pow(2.0, -e.to(torch.float32)).to(torch.float16)
    u = torch.empty(shape, dtype=torch.float32, device=device)
    u.uniform_(0.5, 1.5, generator=g)
    return (u * (w_std / CODE_STD)).to(torch.float16)


def zipf_bias(E: int, s: float, device="cpu") -> torch.Tensor:
    return torch.tensor([-s * math.log(e + 1.0) for e in range(E)],
                        dtype=torch.float32, device=device)


def expert_weights(wl: Workload, e: int, seed: int = 0, device="cpu",
                   pow2_scales: bool = False):
    """(w1[e], w2[e], s1[e], s2[e]) for one expert (scales None if plain)."""
    if wl.wfmt == "int8":
        w1 = int8_codes((wl.d_ff, wl.d), seed, f"w1/{e}", device)
        w2 = int8_codes((wl.d, wl.d_ff), seed, f"w2/{e}", device)
        s1 = fp16_scales((wl.d_ff, wl.d // 128), wl.w_std, seed, f"s1/{e}", device,
                         pow2_scales)
        s2 = fp16_scales((wl.d, wl.d_ff // 128), wl.w_std, seed, f"s2/{e}", device,
                         pow2_scales)
        return w1, w2, s1, s2
    dt = _act_dtype(wl)
    w1 = normal((wl.d_ff, wl.d), wl.w_std, seed, f"w1/{e}", device, dt)
    w2 = normal((wl.d, wl.d_ff), wl.w_std, seed, f"w2/{e}", device, dt)
    return w1, w2, None, None


def make_inputs(wl: Workload, seed: int = 0, device="cpu",
                pow2_scales: bool = False) -> dict:
    """All inputs of one layer call, on ``device``."""
    dt = _act_dtype(wl)
    inp = {
        "x": normal((wl.T, wl.d), wl.x_std, seed, "x", device, dt),
        "w_router": normal((wl.E, wl.d), wl.w_std, seed, "w_router", device, dt),
        "b_router": zipf_bias(wl.E, wl.zipf_s, device) if wl.zipf_s > 0 else None,
    }
    wdt = torch.int8 if wl.wfmt == "int8" else dt
    w1 = torch.empty((wl.E, wl.d_ff, wl.d), dtype=wdt, device=device)
    w2 = torch.empty((wl.E, wl.d, wl.d_ff), dtype=wdt, device=device)
    s1 = s2 = None
    if wl.wfmt == "int8":
        s1 = torch.empty((wl.E, wl.d_ff, wl.d // 128), dtype=torch.float16, device=device)
        s2 = torch.empty((wl.E, wl.d, wl.d_ff // 128), dtype=torch.float16, device=device)
    for e in range(wl.E):
        a, b, c, d = expert_weights(wl, e, seed, device, pow2_scales)
        w1[e].copy_(a)
        w2[e].copy_(b)
        if s1 is not None:
            s1[e].copy_(c)
            s2[e].copy_(d)
    inp.update(w1=w1, w2=w2, w1_scale=s1, w2_scale=s2)
    if wl.pr_moe:
        inp["wm1"] = normal((wl.d_ff_dense, wl.d), wl.w_std, seed, "wm1", device, dt)
        inp["wm2"] = normal((wl.d, wl.d_ff_dense), wl.w_std, seed, "wm2", device, dt)
    else:
        inp["wm1"] = inp["wm2"] = None
    return inp



def router_inputs(wl: Workload, router: str, seed: int = 0, device="cpu",
                  cos_dim: int = 64) -> dict:
    """The extra inputs of a router variant: noisy TopK -> w_noise [E, d]
    (std w_std) and the call's standard-normal draws noise [T, E] fp32;
    cosine -> w_proj [cos_dim, d] (std w_std) and expert_emb [E, cos_dim]
    (std 1).  Seeded like the other inputs; nothing for the other routers."""
    dt = _act_dtype(wl)
    out = {}
    if router == "noisy_topk":
        out["w_noise"] = normal((wl.E, wl.d), wl.w_std, seed, "w_noise", device, dt)
        out["noise"] = normal((wl.T, wl.E), 1.0, seed, "noise", device, torch.float32)
    if router == "cosine":
        out["w_proj"] = normal((cos_dim, wl.d), wl.w_std, seed, "w_proj", device, dt)
        out["expert_emb"] = normal((wl.E, cos_dim), 1.0, seed, "expert_emb", device, dt)
    return out
