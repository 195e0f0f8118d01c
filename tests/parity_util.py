"""Comparison rules between the HIP path and the CPU oracle.

Integers (expert ids, slots, loads, kept counts, drop masks) must match
bit-exactly, except that a token whose k-th and (k+1)-th router logits, as
fp32 values of the oracle's fp64 logits, lie within 1e-5 of each other (a
near-tie) may pick the other expert; such tokens are counted and reported.
Floating outputs: max|a - a_ref| <= tau * max|a_ref| with tau = 1e-4 for
fp32 layers and 2e-2 for bf16 layers, checked separately on the expert rows
(y_disp, kept slots only), the expert term M = sum_j g_j E_j(x), PR-MoE's
dense term D and the output y -- y alone would hide a wrong expert term
behind the residual.  Gates and the aux loss: relative error <= 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

TAU = {"f32": 1e-4, "bf16": 2e-2}
NEAR_TIE = 1e-5


def to_np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.numpy()
    return np.asarray(t)


def near_ties(logits64: np.ndarray, k: int) -> np.ndarray:
    """Indices of tokens whose k-th and (k+1)-th fp32 logits are within 1e-5."""
    E = logits64.shape[1]
    if k >= E:
        return np.zeros(0, np.int64)
    l32 = logits64.astype(np.float32).astype(np.float64)
    srt = -np.sort(-l32, axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    return np.nonzero(gap < NEAR_TIE)[0]


def check_close(name, got, ref, tau, mask=None):
    got = to_np(got).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= tau * max(scale, 1e-30), f"{name}: max err {err:.3e} > {tau} * {scale:.3e}"
    return err / max(scale, 1e-30)


def check_ids(gpu_ids, ref_ids, logits64, k):
    """Bit-exact ids except on reported near-ties; returns (mismatch tokens, near-tie tokens)."""
    g = to_np(gpu_ids)
    r = np.asarray(ref_ids)
    bad = np.nonzero(np.any(g != r, axis=1))[0]
    ties = near_ties(logits64, k)
    assert set(bad.tolist()) <= set(ties.tolist()), (
        f"expert ids differ on tokens that are not near-ties: {sorted(set(bad) - set(ties))[:10]}")
    return bad, ties


def valid_token_order_dispatch(ids, slots, load, kept, C, E):
    """Property check of a dispatch result against its own ids (used when a
    near-tie flipped an id, so the oracle's dispatch no longer applies, and at
    full size); ids < 0 are unused slots."""
    ids, slots = np.asarray(ids), np.asarray(slots)
    T, k = ids.shape
    n = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if e < 0:  # an unused slot (TopP) is no assignment
                assert slots[t, j] == -1
                continue
            want = n[e] if n[e] < C else -1
            assert slots[t, j] == want
            n[e] += 1
    assert np.array_equal(np.asarray(load), n)
    assert np.array_equal(np.asarray(kept), np.minimum(n, C))


def oracle_rows_by_expert(x, inp, want):
    """{e: [token, ...]} -> {e: fp64 [n, d]}: the oracle's expert FFN of the
    rows x[token] through expert e.  x is a CPU tensor; each expert's
    weights (and int8 scales) are moved to the CPU once."""
    import oracle
    out = {}
    s1, s2 = inp.get("w1_scale"), inp.get("w2_scale")
    for e, toks in want.items():
        if len(toks) == 0:
            continue
        out[e] = oracle.ffn_rows(x[list(toks)], inp["w1"][e].cpu(), inp["w2"][e].cpu(),
                                 None if s1 is None else s1[e].cpu(),
                                 None if s2 is None else s2[e].cpu())
    return out


def check_expert_terms(wl, x, inp, ids, slots, gates, y_disp, m, y, tokens, dense=None,
                       tag=""):
    """Element-by-element checks of the expert term on `tokens` under the
    routing (ids, slots, gates: numpy [T, k]) the layer used:
      y_disp[ids[t,j], slots[t,j]] against the oracle FFN of x[t] through
      expert ids[t,j], for every kept (t, j);
      M[t] = sum over kept j of gates[t,j] E_j(x[t])  (the layer's
      moe_combine without bases, `m`);
      y[t] = [x[t]] + [D(x[t])] + M[t]   (dense: fp64 D rows of `tokens`).
    The bound is the workload's tolerance relative to the largest reference
    value of each quantity, so a zeroed or misplaced expert term fails it
    although y's residual is much larger."""
    import oracle
    tau = TAU[wl.act]
    tokens = np.asarray(sorted(set(int(t) for t in tokens)), np.int64)
    n, k = len(tokens), ids.shape[1]
    sl, ii, gg = slots[tokens], ids[tokens], np.asarray(gates, np.float64)[tokens]
    want = {}
    for a, t in enumerate(tokens):
        for j in range(k):
            if sl[a, j] >= 0:
                want.setdefault(int(ii[a, j]), []).append(int(t))
    rows = oracle_rows_by_expert(x, inp, want)
    eo = np.zeros((n, k, wl.d))
    used = {e: 0 for e in want}
    ei, si, at = [], [], []
    for a in range(n):
        for j in range(k):
            if sl[a, j] >= 0:
                e = int(ii[a, j])
                eo[a, j] = rows[e][used[e]]
                used[e] += 1
                ei.append(e)
                si.append(int(sl[a, j]))
                at.append((a, j))
    if ei:
        got = to_np(y_disp[torch.as_tensor(ei, device=y_disp.device),
                           torch.as_tensor(si, device=y_disp.device)])
        ref = np.stack([eo[a, j] for a, j in at])
        check_close(f"y_disp{tag}", got, ref, tau)
    base = np.zeros((n, wl.d))
    if wl.add_skip:
        base += to_np(x[torch.as_tensor(tokens)]).astype(np.float64)
    if dense is not None:
        base += dense
    yref, mref = oracle.combine(sl, gg, eo, base)
    tdev = torch.as_tensor(tokens, device=m.device)
    err_m = check_close(f"M{tag}", m[tdev], mref, tau)
    check_close(f"y{tag}", y[tdev], yref, tau)
    return err_m, len(ei)


GUARD_BYTES = 256
CANARY = 0xA5


def guard_outputs(out):
    """Replace every tensor of a LayerOutputs by one of the same shape and
    type that sits at the start of a larger buffer whose last GUARD_BYTES are
    a canary; returns a function that asserts no canary byte changed (a
    kernel wrote past the end of an output)."""
    import dataclasses
    guards = []
    for f in dataclasses.fields(out):
        t = getattr(out, f.name)
        if not isinstance(t, torch.Tensor):
            continue
        n = t.numel() * t.element_size()
        raw = torch.empty(n + GUARD_BYTES, dtype=torch.uint8, device=t.device)
        raw[n:].fill_(CANARY)
        setattr(out, f.name, raw[:n].view(t.dtype).view(t.shape))
        guards.append((f.name, raw, n))

    def check():
        for name, raw, n in guards:
            tail = raw[n:]
            assert bool((tail == CANARY).all()), f"{name}: bytes written past the end"
    return check
