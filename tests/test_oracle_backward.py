"""Pins of the oracle's layer backward (CPU only).

The backward is checked against the derivative of the (separately pinned)
forward, not against itself: central finite differences of
    L = <dy, y> + g_aux * aux + g_z * z_loss
computed by the oracle's forward on fp64 inputs, for every input element,
at configurations with drops, renormalised top-2 gates, both capacity
policies, PR-MoE and a router bias; and against torch autograd (fp64) on the
one-expert case, where the layer reduces to x + MLP(x) and the z-loss to the
mean squared logit.
"""
import numpy as np
import pytest
import torch

import oracle


def _loss(p, dy, cfg):
    o = oracle.layer_forward(p["x"], p["wr"], p["w1"], p["w2"], k=cfg["k"],
                             capacity_factor=1.0, capacity_override=cfg["C"], bias=p["b"],
                             wm1=p.get("wm1"), wm2=p.get("wm2"), normalize=cfg["normalize"],
                             pr_moe=cfg["pr"], add_skip=cfg["skip"], policy=cfg["policy"],
                             alpha=cfg["alpha"])
    z = oracle.z_loss(o["logits"])
    return float(np.sum(dy * o["y"]) + cfg["g_aux"] * o["aux"] + cfg["g_z"] * z), o


def _params(rng, T, D, E, F, Fd, pr):
    p = dict(x=rng.standard_normal((T, D)), wr=0.5 * rng.standard_normal((E, D)),
             b=(0.3 * rng.standard_normal(E)).astype(np.float32),
             w1=0.4 * rng.standard_normal((E, F, D)), w2=0.4 * rng.standard_normal((E, D, F)))
    if pr:
        p["wm1"] = 0.4 * rng.standard_normal((Fd, D))
        p["wm2"] = 0.4 * rng.standard_normal((D, Fd))
    return p


def _margins_ok(o, k, policy):
    lg = np.sort(o["logits"], axis=1)[:, ::-1]
    if lg.shape[1] > k and np.min(lg[:, k - 1] - lg[:, k]) < 1e-3:
        return False
    if policy == oracle.DROP_GATE_PRIORITY:
        g = np.sort(o["gates"].ravel())
        if np.min(np.diff(g)) < 1e-6:
            return False
    return True


CASES = [
    dict(name="top2_renorm_drops_pr", k=2, normalize=True, policy=oracle.DROP_TOKEN_ORDER,
         pr=True, skip=True, C=4),
    dict(name="top2_gate_priority", k=2, normalize=True, policy=oracle.DROP_GATE_PRIORITY,
         pr=False, skip=True, C=3),
    dict(name="top1_no_skip", k=1, normalize=True, policy=oracle.DROP_TOKEN_ORDER,
         pr=True, skip=False, C=3),
    dict(name="top3_raw_gates", k=3, normalize=False, policy=oracle.DROP_TOKEN_ORDER,
         pr=False, skip=True, C=5),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_backward_matches_finite_differences(case):
    T, D, E, F, Fd = 7, 6, 4, 5, 3
    cfg = dict(case, alpha=0.7, g_aux=0.3, g_z=0.2)
    for seed in range(50):  # a draw whose discrete decisions are not near a flip
        rng = np.random.default_rng(seed)
        p = _params(rng, T, D, E, F, Fd, cfg["pr"])
        dy = rng.standard_normal((T, D))
        _, o = _loss(p, dy, cfg)
        if _margins_ok(o, cfg["k"], cfg["policy"]):
            break
    assert (o["slots"] < 0).any(), "the case must drop some assignments"
    g = oracle.layer_backward(p["x"], p["wr"], p["w1"], p["w2"], dy, k=cfg["k"],
                              capacity_factor=1.0, capacity_override=cfg["C"], bias=p["b"],
                              wm1=p.get("wm1"), wm2=p.get("wm2"), normalize=cfg["normalize"],
                              pr_moe=cfg["pr"], add_skip=cfg["skip"], policy=cfg["policy"],
                              alpha=cfg["alpha"], g_aux=cfg["g_aux"], g_z=cfg["g_z"])
    names = [("x", "dx"), ("wr", "dw_router"), ("w1", "dw1"), ("w2", "dw2"), ("b", "db_router")]
    if cfg["pr"]:
        names += [("wm1", "dwm1"), ("wm2", "dwm2")]
    for pn, gn in names:
        a = p[pn]
        num = np.zeros(a.shape)
        for idx in np.ndindex(a.shape):
            h = 1e-6 if a.dtype == np.float64 else 1e-3
            v = a[idx]
            a[idx] = v + h
            hp = float(a[idx]) - float(v)
            lp, _ = _loss(p, dy, cfg)
            a[idx] = v - h
            hm = float(v) - float(a[idx])
            lm, _ = _loss(p, dy, cfg)
            a[idx] = v
            num[idx] = (lp - lm) / (hp + hm)
        ana = g[gn]
        scale = max(1.0, np.abs(num).max())
        err = np.abs(ana - num).max() / scale
        assert err < 2e-6, f"{gn}: max error {err:.3e} (scale {scale:.3g})"


def test_single_expert_reduces_to_torch_autograd():
    # E = 1: gate = 1 (softmax of one logit), aux = alpha (constant), no drops,
    # z-loss = mean of the squared logit; y = x + W2 GELU(W1 x)
    rng = np.random.default_rng(5)
    T, D, F = 9, 8, 12
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((1, D))
    w1 = 0.5 * rng.standard_normal((1, F, D))
    w2 = 0.5 * rng.standard_normal((1, D, F))
    dy = rng.standard_normal((T, D))
    g_z = 0.4
    g = oracle.layer_backward(x, wr, w1, w2, dy, k=1, capacity_factor=1.0, add_skip=True,
                              alpha=0.9, g_aux=0.5, g_z=g_z)
    tx, twr, tw1, tw2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                         for a in (x, wr, w1[0], w2[0]))
    y = tx + torch.nn.functional.gelu(tx @ tw1.T) @ tw2.T
    L = (torch.tensor(dy) * y).sum() + g_z * ((tx @ twr.T) ** 2).mean()
    L.backward()
    for ana, ref in ((g["dx"], tx.grad), (g["dw_router"], twr.grad), (g["dw1"][0], tw1.grad),
                     (g["dw2"][0], tw2.grad)):
        np.testing.assert_allclose(ana, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_sampled_entries_equal_the_full_backward(case):
    # the restricted chain rule (used at full size) against the whole backward
    T, D, E, F, Fd = 9, 6, 4, 5, 3
    rng = np.random.default_rng(11)
    p = _params(rng, T, D, E, F, Fd, case["pr"])
    dy = rng.standard_normal((T, D))
    kw = dict(k=case["k"], bias=p["b"], wm1=p.get("wm1"), wm2=p.get("wm2"),
              normalize=case["normalize"], pr_moe=case["pr"], add_skip=case["skip"],
              alpha=0.7, g_aux=0.3, g_z=0.2)
    fw = oracle.layer_forward(p["x"], p["wr"], p["w1"], p["w2"], capacity_factor=1.0,
                              capacity_override=case["C"], policy=case["policy"],
                              **{k: v for k, v in kw.items() if k not in ("g_aux", "g_z")})
    full = oracle.layer_backward(p["x"], p["wr"], p["w1"], p["w2"], dy, capacity_factor=1.0,
                                 capacity_override=case["C"], policy=case["policy"], **kw)
    i1 = [(e, f, i) for e in range(E) for f in range(F) for i in range(D)]
    i2 = [(e, o, f) for e in range(E) for o in range(D) for f in range(F)]
    s = oracle.backward_sampled(p["x"], p["wr"], p["w1"], p["w2"], fw["ids"], fw["slots"], dy,
                                np.arange(T), dw1_idx=i1, dw2_idx=i2, **kw)
    np.testing.assert_allclose(s["dx"], full["dx"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s["dw1"], full["dw1"].ravel(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s["dw2"], full["dw2"].ravel(), rtol=1e-11, atol=1e-12)
