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
