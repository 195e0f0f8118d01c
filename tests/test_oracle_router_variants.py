"""Pins of the oracle's router variants (CPU only).

TopP selection, the cosine router, noisy TopK gating and the Importance /
Load CoV^2 losses (survey notes secs. 1.1.1.1, 1.1.1.2, 1.1.4.1, 1.1.4.2)
are checked against what fixes them independently of their code: reductions
to the separately pinned softmax router, closed forms, invariances, the
defining properties of the TopP set, a Monte Carlo estimate of the Load
probability, and numpy's variance.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle

R = oracle


def _xw(seed, T=12, d=16, E=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w = 0.5 * rng.standard_normal((E, d))
    b = (0.2 * rng.standard_normal(E)).astype(np.float32)
    return rng, x, w, b


@pytest.mark.parametrize("k,normalize", [(1, True), (2, True), (3, False)])
def test_topk_variant_is_the_softmax_router(k, normalize):
    _, x, w, b = _xw(0)
    v = oracle.route_variant(x, w, k, router=R.ROUTER_TOPK, bias=b, normalize=normalize)
    r = oracle.route(x, w, k, bias=b, normalize=normalize)
    assert np.array_equal(v["ids"], r["ids"])
    np.testing.assert_array_equal(v["gates"], r["gates"])
    np.testing.assert_array_equal(v["logits"], r["logits"])
    member = np.zeros_like(v["load_p"])
    np.put_along_axis(member, r["ids"].astype(np.int64), 1.0, axis=1)
    np.testing.assert_array_equal(v["load_p"], member)


# ------------------------------------------------------------------ TopP
@pytest.mark.parametrize("normalize", [True, False])
def test_top_p_tiny_threshold_takes_one_expert(normalize):
    _, x, w, b = _xw(1)
    v = oracle.route_variant(x, w, 4, router=R.ROUTER_TOP_P, bias=b, top_p=1e-12,
                             normalize=normalize)
    r = oracle.route(x, w, 1, bias=b)
    assert np.array_equal(v["ids"][:, 0], r["ids"][:, 0])
    assert (v["ids"][:, 1:] == -1).all() and (v["gates"][:, 1:] == 0).all()
    np.testing.assert_allclose(v["gates"][:, 0], 1.0 if normalize else r["gates"][:, 0],
                               rtol=1e-15)


def test_top_p_of_one_is_renormalised_topk():
    # the cumulative probability of k < E experts stays below 1
    _, x, w, b = _xw(2)
    v = oracle.route_variant(x, w, 3, router=R.ROUTER_TOP_P, bias=b, top_p=1.0)
    r = oracle.route(x, w, 3, bias=b, normalize=True)
    assert np.array_equal(v["ids"], r["ids"])
    np.testing.assert_allclose(v["gates"], r["gates"], rtol=1e-14)


def test_top_p_two_experts_closed_form():
    # E = 2: the leader has p = sigmoid(|l0 - l1|); one expert iff that exceeds P
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 4))
    w = rng.standard_normal((2, 4))
    lg = x @ w.T
    pmax = expit(np.abs(lg[:, 0] - lg[:, 1]))
    for P in (0.55, 0.7, 0.9, 0.97):
        ok = np.abs(pmax - P) > 1e-9
        v = oracle.route_variant(x, w, 2, router=R.ROUTER_TOP_P, top_p=P)
        n = (v["ids"] >= 0).sum(1)
        assert np.array_equal(n[ok], np.where(pmax[ok] > P, 1, 2)[ok])


@pytest.mark.parametrize("P", [0.3, 0.6, 0.85])
def test_top_p_set_properties(P):
    # the taken set: the most probable experts (a prefix of the order), whose
    # mass exceeds P unless the k slots ran out, and minimal with that mass
    _, x, w, b = _xw(4, T=50, E=8)
    k = 5
    v = oracle.route_variant(x, w, k, router=R.ROUTER_TOP_P, bias=b, top_p=P, normalize=False)
    p = v["probs"]
    for t in range(x.shape[0]):
        S = [int(e) for e in v["ids"][t] if e >= 0]
        n = len(S)
        assert 1 <= n <= k and len(set(S)) == n
        assert (v["ids"][t, n:] == -1).all()
        outside = [e for e in range(p.shape[1]) if e not in S]
        assert min(p[t, S]) >= max(p[t, outside])
        mass = p[t, S].sum()
        assert mass > P or n == k
        assert p[t, S].sum() - min(p[t, S]) <= P
        np.testing.assert_allclose(v["gates"][t, :n], p[t, S], rtol=1e-15)


# ------------------------------------------------------------------ cosine
def test_cosine_identity_projection_closed_form():
    # W_proj = I, expert embeddings = unit rows: logit_e = x_e / (tau |x|)
    rng = np.random.default_rng(5)
    d = 6
    x = rng.standard_normal((9, d))
    tau = 0.35
    v = oracle.route_variant(x, np.eye(d), 2, router=R.ROUTER_COSINE, emb=np.eye(d), tau=tau)
    ref = x / (tau * np.linalg.norm(x, axis=1, keepdims=True))
    np.testing.assert_allclose(v["logits"], ref, rtol=1e-13)


def test_cosine_invariances_and_reduction():
    rng = np.random.default_rng(6)
    T, d, de, E = 15, 12, 5, 7
    x = rng.standard_normal((T, d))
    wp = rng.standard_normal((de, d))
    emb = rng.standard_normal((E, de))
    tau = 0.2
    base = oracle.route_variant(x, wp, 2, router=R.ROUTER_COSINE, emb=emb, tau=tau)
    # scaling a token or an expert embedding by a positive factor changes nothing
    s = oracle.route_variant(3.0 * x, wp, 2, router=R.ROUTER_COSINE,
                             emb=emb * rng.uniform(0.5, 4.0, (E, 1)), tau=tau)
    np.testing.assert_allclose(s["logits"], base["logits"], rtol=1e-12)
    # halving tau doubles the logits; they lie in [-1/tau, 1/tau]
    h = oracle.route_variant(x, wp, 2, router=R.ROUTER_COSINE, emb=emb, tau=tau / 2)
    np.testing.assert_allclose(h["logits"], 2 * base["logits"], rtol=1e-13)
    assert np.abs(base["logits"]).max() <= 1 / tau + 1e-12
    # = the (pinned) linear router on the unit projection with W = unit embeddings / tau
    u = x @ wp.T
    un = u / np.linalg.norm(u, axis=1, keepdims=True)
    wn = emb / np.linalg.norm(emb, axis=1, keepdims=True) / tau
    lin = oracle.route(un, wn, 2)
    np.testing.assert_allclose(base["logits"], lin["logits"], rtol=1e-12, atol=1e-13)
    assert np.array_equal(base["ids"], lin["ids"])
    np.testing.assert_allclose(base["gates"], lin["gates"], rtol=1e-12)


def test_cosine_zero_token_gives_the_bias():
    x = np.zeros((2, 4))
    b = np.array([0.5, -1.0, 0.25], np.float32)
    v = oracle.route_variant(x, np.ones((3, 4)), 1, router=R.ROUTER_COSINE,
                             emb=np.ones((3, 3)), tau=0.5, bias=b)
    np.testing.assert_array_equal(v["logits"], np.tile(b.astype(np.float64), (2, 1)))


# ------------------------------------------------------------------ noisy
@pytest.mark.parametrize("k", [1, 2, 3])
def test_noisy_without_noise_is_the_softmax_router(k):
    rng, x, w, b = _xw(7)
    wn = rng.standard_normal(w.shape)
    v = oracle.route_variant(x, w, k, router=R.ROUTER_NOISY, bias=b, w_noise=wn,
                             noise=np.zeros((x.shape[0], w.shape[0]), np.float32))
    r = oracle.route(x, w, k, bias=b, normalize=True)
    np.testing.assert_array_equal(v["logits"], r["logits"])
    assert np.array_equal(v["ids"], r["ids"])
    # the gates are the softmax over the kept scores: 1 for k = 1
    np.testing.assert_allclose(v["gates"], 1.0 if k == 1 else r["gates"], rtol=1e-14)


def test_noisy_scale_of_zero_noise_weights_is_log2():
    rng, x, w, b = _xw(8)
    eps = rng.standard_normal((x.shape[0], w.shape[0])).astype(np.float32)
    v = oracle.route_variant(x, w, 2, router=R.ROUTER_NOISY, bias=b,
                             w_noise=np.zeros_like(w), noise=eps)
    clean = oracle.route(x, w, 2, bias=b)["logits"]
    np.testing.assert_allclose(v["logits"], clean + eps.astype(np.float64) * np.log(2.0),
                               rtol=1e-13, atol=1e-14)


def test_noisy_load_probability_by_monte_carlo():
    # P(x, e): redraw e's noise alone, everything else held; is e in the TopK?
    rng = np.random.default_rng(9)
    T, d, E, k = 3, 8, 5, 2
    x = rng.standard_normal((T, d))
    w = 0.4 * rng.standard_normal((E, d))
    wn = 0.4 * rng.standard_normal((E, d))
    eps = rng.standard_normal((T, E)).astype(np.float32)
    v = oracle.route_variant(x, w, k, router=R.ROUTER_NOISY, w_noise=wn, noise=eps)
    clean = x @ w.T
    sig = np.log1p(np.exp(x @ wn.T))
    H = clean + eps * sig
    n = 200_000
    for t in range(T):
        for e in range(E):
            draws = rng.standard_normal(n)
            He = clean[t, e] + draws * sig[t, e]
            others = np.sort(np.delete(H[t], e))[::-1]
            frac = np.mean(He > others[k - 1])
            pe = v["load_p"][t, e]
            assert abs(frac - pe) <= 4 * np.sqrt(max(pe * (1 - pe), 1e-6) / n) + 1e-3, (t, e)


def test_noisy_load_probability_is_one_when_every_expert_is_kept():
    rng, x, w, b = _xw(10, E=3)
    v = oracle.route_variant(x, w, 3, router=R.ROUTER_NOISY, w_noise=rng.standard_normal(w.shape),
                             noise=rng.standard_normal((x.shape[0], 3)).astype(np.float32))
    np.testing.assert_array_equal(v["load_p"], 1.0)


# ------------------------------------------------------------------ losses
def test_cov2_closed_forms_and_numpy():
    assert oracle.cov2(np.full(7, 3.5)) == 0.0
    for E in (2, 5, 64):
        v = np.zeros(E)
        v[3 % E] = 11.0
        np.testing.assert_allclose(oracle.cov2(v), E - 1, rtol=1e-14)
    rng = np.random.default_rng(11)
    v = rng.uniform(0.1, 5.0, 40)
    np.testing.assert_allclose(oracle.cov2(v), np.var(v) / np.mean(v) ** 2, rtol=1e-13)
    assert oracle.cov2(np.zeros(4)) == 0.0


@pytest.mark.parametrize("router", [R.ROUTER_TOPK, R.ROUTER_TOP_P, R.ROUTER_COSINE,
                                    R.ROUTER_NOISY])
def test_importance_and_load_totals(router):
    rng, x, w, b = _xw(12, T=30, E=6)
    kw = dict(router=router, bias=b, normalize=True, top_p=0.7, tau=0.3)
    if router == R.ROUTER_NOISY:
        kw.update(w_noise=rng.standard_normal(w.shape),
                  noise=rng.standard_normal((30, 6)).astype(np.float32))
    if router == R.ROUTER_COSINE:
        kw.update(emb=rng.standard_normal((6, 5)))
        w = rng.standard_normal((5, x.shape[1]))
    k = 3
    v = oracle.route_variant(x, w, k, **kw)
    valid = v["ids"] >= 0
    # renormalised (or TopK-then-softmax) gates sum to 1 per token
    np.testing.assert_allclose(v["importance"].sum(), x.shape[0], rtol=1e-12)
    if router != R.ROUTER_NOISY:
        np.testing.assert_allclose(v["load"].sum(), valid.sum(), rtol=0)
    for e in range(6):
        np.testing.assert_allclose(v["importance"][e], v["gates"][v["ids"] == e].sum(),
                                   rtol=1e-13)


# ------------------------------------------------------------------ layer
def test_layer_with_top_p_composes_the_stages():
    rng = np.random.default_rng(13)
    T, D, E, F, k = 20, 8, 4, 6, 3
    x = rng.standard_normal((T, D)).astype(np.float32)
    wr = rng.standard_normal((E, D)).astype(np.float32)
    w1 = (0.3 * rng.standard_normal((E, F, D))).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((E, D, F))).astype(np.float32)
    o = oracle.layer_forward(x, wr, w1, w2, k=k, capacity_factor=0.5, router=R.ROUTER_TOP_P,
                             top_p=0.6)
    r = oracle.route_variant(x, wr, k, router=R.ROUTER_TOP_P, top_p=0.6)
    assert np.array_equal(o["ids"], r["ids"]) and (o["ids"] == -1).any()
    C = o["capacity"]
    dsp = oracle.dispatch(r["ids"], E, C)
    assert np.array_equal(o["slots"], dsp["slots"])
    assert (dsp["drop"][r["ids"] < 0] == 0).all() and (dsp["slots"][r["ids"] < 0] == -1).all()
    assert np.array_equal(dsp["load"], np.bincount(r["ids"][r["ids"] >= 0], minlength=E))
    eo = np.zeros((T, k, D))
    for t in range(T):
        for j in range(k):
            if dsp["slots"][t, j] >= 0:
                e = r["ids"][t, j]
                eo[t, j] = oracle.ffn_rows(x[t], w1[e], w2[e])[0]
    y, _ = oracle.combine(dsp["slots"], r["gates"], eo, base=x.astype(np.float64))
    np.testing.assert_allclose(o["y"], y, rtol=1e-13, atol=1e-13)
