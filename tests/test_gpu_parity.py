"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small shapes compare every output element by element; they span several
tiles and a ragged tail.  The five workloads at full size run in the launch
configuration the benchmark times (moe_layer_forward) and are compared on
all routing outputs plus sampled expert rows and tokens, which the oracle
computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_24_amd import binding, synth, workloads
from parity_util import (TAU, check_close, check_expert_terms, check_ids, guard_outputs,
                         oracle_rows_by_expert, to_np, valid_token_order_dispatch)

pytestmark = pytest.mark.gpu

W = workloads.Workload
DEV = "cuda"


def _cpu(inp):
    return {k: (None if v is None else v.cpu()) for k, v in inp.items()}


def _run_layer(wl, inp, overlap_dense=True, **alloc):
    cfg = binding.config_of(wl, overlap_dense=overlap_dense)
    out = binding.alloc_outputs(cfg, DEV, logits=True, x_disp=True, y_disp=True,
                                dense_out=True, **alloc)
    check_guards = guard_outputs(out)  # canaries past the end of every output
    ws = binding.alloc_workspace(cfg)
    binding.moe_layer_forward(cfg, inp["x"], inp, out, ws)
    m = torch.empty_like(out.y)
    binding.moe_combine(cfg, out.y_disp, out.expert_ids, out.slots, out.gates, None, None, m)
    torch.cuda.synchronize()
    check_guards()
    return cfg, out, m


def _oracle_layer(wl, ic):
    return oracle.layer_forward(
        ic["x"], ic["w_router"], ic["w1"], ic["w2"], k=wl.k,
        capacity_factor=wl.capacity_factor, bias=ic["b_router"], s1=ic["w1_scale"],
        s2=ic["w2_scale"], wm1=ic["wm1"], wm2=ic["wm2"], normalize=wl.normalize_topk,
        pr_moe=wl.pr_moe, add_skip=wl.add_skip, alpha=wl.aux_alpha)


def _check_routing(wl, out, ref, C):
    bad, ties = check_ids(out.expert_ids, ref["ids"], ref["logits"], wl.k)
    if len(ties):
        print(f"[{wl.name}] near-tie tokens: {len(ties)} {ties[:8].tolist()}; flipped: {bad.tolist()}")
    ok = np.ones(wl.T, bool)
    ok[bad] = False
    check_close("gates", out.gates, ref["gates"], 1e-5, mask=ok)
    scale = max(1.0, float(np.abs(ref["logits"]).max()))
    assert np.abs(to_np(out.logits) - ref["logits"]).max() <= 1e-5 * scale
    aux = float(to_np(out.aux_loss)[0])
    assert aux == pytest.approx(ref["aux"], rel=1e-5, abs=1e-7)
    if len(bad) == 0:
        assert np.array_equal(to_np(out.slots), ref["slots"])
        assert np.array_equal(to_np(out.drop_mask), ref["drop"])
        assert np.array_equal(to_np(out.load), ref["load"])
        assert np.array_equal(to_np(out.kept), ref["kept"])
    else:
        valid_token_order_dispatch(to_np(out.expert_ids), to_np(out.slots), to_np(out.load),
                                   to_np(out.kept), C, wl.E)
    return bad


# ------------------------------------------------------------ whole layer, small
SMALL = [
    workloads.WORKLOADS["tiny_f32"],
    W("f32_top2_ragged", T=77, d=24, E=5, k=2, d_ff=40, capacity_factor=1.0, act="f32",
      w_std=0.2),
    W("moe128_350m_small", T=520, d=256, E=16, k=1, d_ff=512, capacity_factor=1.0),
    W("prmoe_small", T=300, d=256, E=8, k=1, d_ff=512, capacity_factor=1.0,
      d_ff_dense=512, pr_moe=True, add_skip=False),
    W("prmoe_small_skip", T=130, d=128, E=6, k=1, d_ff=256, capacity_factor=0.5,
      d_ff_dense=384, pr_moe=True, add_skip=True),
    W("decode_small", T=32, d=256, E=8, k=2, d_ff=384, capacity_factor=4.0),
    W("skewed_int8_small", T=700, d=256, E=8, k=2, d_ff=512, capacity_factor=1.25,
      wfmt="int8", zipf_s=1.2),
    W("top3_bigE", T=333, d=128, E=200, k=3, d_ff=128, capacity_factor=2.0),
    # degenerate routings: one expert (C = T, nothing dropped, gate 1), every
    # token to every expert (k = E), the largest E and k the library takes
    W("one_expert", T=100, d=128, E=1, k=1, d_ff=256, capacity_factor=1.0),
    W("k_equals_E", T=90, d=128, E=4, k=4, d_ff=128, capacity_factor=1.0),
    W("max_E_k_plain_gates", T=256, d=128, E=256, k=8, d_ff=128, capacity_factor=1.0,
      normalize_topk=False),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_layer_small_all_outputs(wl):
    print(f"[layer_small] {wl}", flush=True)
    inp = synth.make_inputs(wl, seed=1)
    ref = _oracle_layer(wl, inp)
    dinp = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    cfg, out, m = _run_layer(wl, dinp)
    C = binding.capacity(cfg)
    assert C == ref["capacity"]
    bad = _check_routing(wl, out, ref, C)
    assert len(bad) == 0
    tau = TAU[wl.act]
    # expert rows, kept slots only
    yd = to_np(out.y_disp)
    xd = to_np(out.x_disp)
    x = to_np(inp["x"])
    for t in range(wl.T):
        for j in range(wl.k):
            s = ref["slots"][t, j]
            if s >= 0:
                e = ref["ids"][t, j]
                assert np.array_equal(xd[e, s], x[t])  # gather is an exact copy
    mask = np.zeros((wl.T, wl.k), bool)
    mask[ref["slots"] >= 0] = True
    got_rows = np.zeros((wl.T, wl.k, wl.d))
    for t, j in zip(*np.nonzero(mask)):
        got_rows[t, j] = yd[ref["ids"][t, j], ref["slots"][t, j]]
    check_close("y_disp", got_rows[mask], ref["expert_out"][mask], tau)
    check_close("M", m, ref["m"], tau)
    if wl.pr_moe:
        check_close("D", out.dense_out, ref["dense"], tau)
    check_close("y", out.y, ref["y"], tau)


# ------------------------------------------------------------ entry points alone
@pytest.mark.parametrize("act,T,d,E,k,bias", [
    ("f32", 64, 32, 4, 1, False), ("f32", 100, 40, 7, 2, True),
    ("bf16", 100, 128, 5, 1, False), ("bf16", 300, 256, 64, 2, False),
    ("bf16", 257, 128, 128, 1, True), ("bf16", 130, 64, 200, 3, False),
    ("bf16", 65, 64, 256, 2, True), ("bf16", 1, 64, 32, 1, False),
    # eight-wave fused router with three 64-expert slots per lane
    ("bf16", 257, 128, 160, 2, True),
    # split K (at most 16 token blocks, d >= 512): partial products, then the
    # split sums and the epilogue in one kernel; one to four expert slots per
    # lane, k up to 8, partly filled token blocks, a single token
    ("bf16", 32, 1024, 64, 2, True), ("bf16", 65, 512, 160, 3, False),
    ("bf16", 300, 1024, 256, 8, True), ("bf16", 1, 512, 128, 1, False)])
def test_route_alone(act, T, d, E, k, bias):
    wl = W("r", T=T, d=d, E=E, k=k, d_ff=64, capacity_factor=1.0, act=act,
           zipf_s=1.2 if bias else 0.0, w_std=0.1)
    inp = synth.make_inputs(wl, seed=3)
    ref = oracle.route(inp["x"], inp["w_router"], k, bias=inp["b_router"])
    cfg = binding.config_of(wl)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    aux = torch.empty(1, dtype=torch.float32, device=DEV)
    b = None if inp["b_router"] is None else inp["b_router"].to(DEV)
    binding.moe_route(cfg, inp["x"].to(DEV), inp["w_router"].to(DEV), b, ids, gates, logits,
                      aux, binding.alloc_workspace(cfg, binding.ENTRY_ROUTE))
    torch.cuda.synchronize()
    bad, _ = check_ids(ids, ref["ids"], ref["logits"], k)
    assert len(bad) == 0
    check_close("gates", gates, ref["gates"], 1e-5)
    loss, _, _ = oracle.aux_loss(ref["ids"], ref["probs"], 1.0)
    assert float(aux.item()) == pytest.approx(loss, rel=1e-5)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_route_exact_ties_break_to_lower_index(k):
    # zero router: every logit is exactly 0 -> experts 0..k-1 in order
    T, d, E = 70, 64, 6
    cfg = binding.make_config(T=T, d=d, E=E, k=k, d_ff=64)
    x = synth.normal((T, d), 1.0, 0, "x", DEV, torch.bfloat16)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
    aux = torch.empty(1, dtype=torch.float32, device=DEV)
    binding.moe_route(cfg, x, torch.zeros(E, d, dtype=torch.bfloat16, device=DEV), None, ids,
                      gates, None, aux, binding.alloc_workspace(cfg, binding.ENTRY_ROUTE))
    torch.cuda.synchronize()
    assert to_np(ids).tolist() == [list(range(k))] * T
    g = 1.0 / E if k == 1 else 1.0 / k
    assert np.all(to_np(gates) == np.float32(g))
    assert float(aux.item()) == pytest.approx(1.0, abs=1e-6)
    # integer logits with planted ties: one-hot tokens, small-integer router
    rng = np.random.default_rng(k)
    T2 = d
    lg = rng.integers(-2, 3, size=(T2, E)).astype(np.float32)
    xo = np.eye(T2, d, dtype=np.float32)
    wr = lg.T.copy()  # [E, d]: logits[t, e] = lg[t, e]
    ref = oracle.route(xo, wr, k)
    cfg2 = binding.make_config(T=T2, d=d, E=E, k=k, d_ff=64)
    ids2 = torch.empty(T2, k, dtype=torch.int32, device=DEV)
    binding.moe_route(cfg2, torch.from_numpy(xo).to(DEV, torch.bfloat16),
                      torch.from_numpy(wr).to(DEV, torch.bfloat16), None, ids2,
                      torch.empty(T2, k, dtype=torch.float32, device=DEV), None,
                      torch.empty(1, dtype=torch.float32, device=DEV),
                      binding.alloc_workspace(cfg2, binding.ENTRY_ROUTE))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(ids2), ref["ids"])


# holes: share of the ids set outside [0, E) (-1, as a TopP router leaves an
# unused slot, or E): no assignment, counted nowhere
@pytest.mark.parametrize("T,E,k,C,holes", [(1000, 7, 2, 150, 0), (64 * 5 + 3, 128, 1, 3, 0),
                                           (50, 3, 3, 50, 0), (200, 16, 2, 1, 0),
                                           (129, 256, 1, 2, 0), (300, 200, 8, 20, 0),
                                           (777, 192, 3, 16, 0.1), (500, 65, 2, 40, 0.05),
                                           (70, 256, 4, 3, 0.2), (64, 1, 1, 64, 0.3)])
def test_dispatch_alone(T, E, k, C, holes):
    d = 128
    rng = np.random.default_rng(T + E)
    # skewed synthetic choices: distinct experts per token
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    if holes:
        hole = rng.random(ids.shape) < holes
        ids[hole] = np.where(rng.random(ids.shape) < 0.5, -1, E)[hole]
        assert hole.any()
    ref = oracle.dispatch(ids, E, C)
    cfg = binding.make_config(T=T, d=d, E=E, k=k, d_ff=64, capacity=C)
    assert binding.capacity(cfg) == C
    x = synth.normal((T, d), 1.0, 5, "x", DEV, torch.bfloat16)
    slots = torch.empty(T, k, dtype=torch.int32, device=DEV)
    drop = torch.empty(T, k, dtype=torch.uint8, device=DEV)
    load = torch.empty(E, dtype=torch.int32, device=DEV)
    kept = torch.empty(E, dtype=torch.int32, device=DEV)
    xd = torch.full((E, C, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    binding.moe_dispatch(cfg, x, torch.from_numpy(ids).to(DEV), slots, drop, load, kept, xd,
                         binding.alloc_workspace(cfg, binding.ENTRY_DISPATCH))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(slots), ref["slots"])
    assert np.array_equal(to_np(drop), ref["drop"])
    assert np.array_equal(to_np(load), ref["load"])
    assert np.array_equal(to_np(kept), ref["kept"])
    xn, xdn = to_np(x), to_np(xd)
    for t in range(T):
        for j in range(k):
            if ref["slots"][t, j] >= 0:
                assert np.array_equal(xdn[ids[t, j], ref["slots"][t, j]], xn[t])


# (C, d, d_ff): weight-streaming tiles for C <= 32 / 64 / 128 (128x512 when N
# is a multiple of 512, else 128x256 or 128x128), 256x256 and 128x128 block
# tiles above, the 16x64 tile when N is not a multiple of 128
FFN_CASES = [(10, 128, 256), (20, 128, 256), (50, 128, 256), (100, 256, 384), (128, 128, 128),
             (90, 512, 768),
             (300, 256, 512), (200, 384, 384), (40, 192, 320),
             # K a multiple of 1024: the DMA int8 tiles (256- and 128-row), partial tiles
             (300, 1024, 1024), (100, 1024, 2048)]


# int8 groups need d and d_ff multiples of 128 (other shapes are rejected:
# tests/test_abi_cpu.py)
@pytest.mark.parametrize("C,d,F,wfmt", [
    (C, d, F, w) for (C, d, F) in FFN_CASES for w in ("plain", "int8")
    if w == "plain" or (d % 128 == 0 and F % 128 == 0)])
def test_expert_ffn_alone(C, d, F, wfmt):
    E = 4
    wl = W("f", T=C, d=d, E=E, k=1, d_ff=F, capacity_factor=float(E), wfmt=wfmt)
    cfg = binding.config_of(wl)
    assert binding.capacity(cfg) == C
    inp = synth.make_inputs(wl, seed=7)
    rng = np.random.default_rng(C)
    kept = np.array([C, 0, int(rng.integers(1, C + 1)), max(1, C // 3)], np.int32)
    xd = synth.normal((E, C, d), 1.0, 8, "xd", "cpu", torch.bfloat16)
    yd = torch.full((E, C, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    binding.moe_expert_ffn(cfg, xd.to(DEV), torch.from_numpy(kept).to(DEV),
                           inp["w1"].to(DEV), None if inp["w1_scale"] is None else inp["w1_scale"].to(DEV),
                           inp["w2"].to(DEV), None if inp["w2_scale"] is None else inp["w2_scale"].to(DEV),
                           yd, binding.alloc_workspace(cfg, binding.ENTRY_EXPERT_FFN))
    torch.cuda.synchronize()
    ydn = to_np(yd)
    for e in range(E):
        n = kept[e]
        if n == 0:
            continue
        s1 = None if inp["w1_scale"] is None else inp["w1_scale"][e]
        s2 = None if inp["w2_scale"] is None else inp["w2_scale"][e]
        ref = oracle.ffn_rows(xd[e, :n], inp["w1"][e], inp["w2"][e], s1, s2)
        check_close(f"y_disp[{e}]", ydn[e, :n], ref, TAU["bf16"])
    # rows past kept[e] are not written
    assert np.all(np.isnan(ydn[1]))
    assert np.all(np.isnan(ydn[3, kept[3]:]))


@pytest.mark.parametrize("E,C,F", [(40, 300, 1024), (32, 200, 768), (256, 136, 512)])
def test_int8_expert_schedule_matches_unscheduled_tiles(E, C, F):
    # int8 experts with C > 128 run on the XCD schedule (skewed loads, empty
    # and single-row experts, light experts (<= 64 rows; not when d_ff is not
    # a multiple of 512), tiles with one or two busy row bands, one and two
    # 256-row tiles; E at both ends of the schedule's range); the same
    # experts eight at a time take the unscheduled tile order.  Same tiles,
    # same arithmetic: bit-identical rows.  Sampled rows against the oracle.
    d = 1024
    wl = W("s", T=C, d=d, E=E, k=1, d_ff=F, capacity_factor=float(E), wfmt="int8")
    cfg = binding.config_of(wl)
    assert binding.capacity(cfg) == C
    inp = synth.make_inputs(wl, seed=5)
    head = [C, C, 0, 1, min(256, C), min(257, C), min(255, C), 3, 128, 129, 64, 65]
    kept = np.array((head + [int(C * 0.8 ** i) for i in range(E)])[:E], np.int32)
    xd = synth.normal((E, C, d), 1.0, 9, "xd", "cpu", torch.bfloat16)
    w1, s1, w2, s2 = (inp[n].to(DEV) for n in ("w1", "w1_scale", "w2", "w2_scale"))
    ys = torch.full((E, C, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    binding.moe_expert_ffn(cfg, xd.to(DEV), torch.from_numpy(kept).to(DEV), w1, s1, w2, s2, ys,
                           binding.alloc_workspace(cfg, binding.ENTRY_EXPERT_FFN))
    w8 = W("s8", T=C, d=d, E=8, k=1, d_ff=F, capacity_factor=8.0, wfmt="int8")
    cfg8 = binding.config_of(w8)
    ws8 = binding.alloc_workspace(cfg8, binding.ENTRY_EXPERT_FFN)
    yu = torch.full((E, C, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    for e0 in range(0, E, 8):
        sl = slice(e0, e0 + 8)
        binding.moe_expert_ffn(cfg8, xd[sl].to(DEV), torch.from_numpy(kept[sl].copy()).to(DEV),
                               w1[sl], s1[sl], w2[sl], s2[sl], yu[sl], ws8)
    torch.cuda.synchronize()
    for e in range(E):
        n = int(kept[e])
        assert torch.equal(ys[e, :n], yu[e, :n]), f"expert {e}"
        assert torch.isnan(ys[e, n:].float()).all(), f"expert {e}: rows past kept written"
    rng = np.random.default_rng(3)
    for e in (0, 3, 5, 9, 12):
        n = int(kept[e])
        rows = sorted({0, n - 1, *rng.integers(0, n, size=3).tolist()})
        ref = oracle.ffn_rows(xd[e, rows], inp["w1"][e], inp["w2"][e], inp["w1_scale"][e],
                              inp["w2_scale"][e])
        check_close(f"y_disp[{e}]", ys[e, rows], ref, TAU["bf16"])


# (700, 512, 4096): three row tiles (the last ragged) by 16 column tiles,
# the dense MLP's row groups of 2 with a partial last group
@pytest.mark.parametrize("T,d,Fd", [(300, 256, 512), (1000, 256, 512), (17, 64, 128),
                                    (700, 512, 4096)])
def test_dense_mlp_alone(T, d, Fd):
    wl = W("dm", T=T, d=d, E=2, k=1, d_ff=64, capacity_factor=1.0, d_ff_dense=Fd, pr_moe=True)
    cfg = binding.config_of(wl)
    x = synth.normal((T, d), 1.0, 1, "x", "cpu", torch.bfloat16)
    wm1 = synth.normal((Fd, d), 0.02, 1, "wm1", "cpu", torch.bfloat16)
    wm2 = synth.normal((d, Fd), 0.02, 1, "wm2", "cpu", torch.bfloat16)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=DEV)
    binding.moe_dense_mlp(cfg, x.to(DEV), wm1.to(DEV), wm2.to(DEV), out,
                          binding.alloc_workspace(cfg))
    torch.cuda.synchronize()
    check_close("D", out, oracle.ffn_rows(x, wm1, wm2), TAU["bf16"])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_combine_alone(act):
    T, E, k, C = 150, 5, 2, 40
    d = 96 if act == "f32" else 128
    rng = np.random.default_rng(2)
    dt = torch.float32 if act == "f32" else torch.bfloat16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    slots = rng.integers(-1, C, size=(T, k)).astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    yd = synth.normal((E, C, d), 1.0, 2, "yd", "cpu", dt)
    base = synth.normal((T, d), 1.0, 2, "b", "cpu", dt)
    base2 = synth.normal((T, d), 1.0, 2, "b2", "cpu", dt)
    ydn = yd.double().numpy()
    eo = np.zeros((T, k, d))
    for t in range(T):
        for j in range(k):
            if slots[t, j] >= 0:
                eo[t, j] = ydn[ids[t, j], slots[t, j]]
    cfg = binding.make_config(T=T, d=d, E=E, k=k, d_ff=64, capacity=C, act=act)
    y = torch.empty(T, d, dtype=dt, device=DEV)
    y0 = torch.empty(T, d, dtype=dt, device=DEV)
    args = (torch.from_numpy(ids).to(DEV), torch.from_numpy(slots).to(DEV),
            torch.from_numpy(gates).to(DEV))
    binding.moe_combine(cfg, yd.to(DEV), *args, base.to(DEV), base2.to(DEV), y)
    binding.moe_combine(cfg, yd.to(DEV), *args, None, None, y0)
    torch.cuda.synchronize()
    ref, m = oracle.combine(slots, gates.astype(np.float64), eo,
                            base.double().numpy() + base2.double().numpy())
    check_close("y", y, ref, TAU[act])
    check_close("M", y0, m, TAU[act])


# ------------------------------------------------------------ properties
def test_layer_is_deterministic_and_ignores_unwritten_rows():
    wl = SMALL[2]
    inp = {k: (None if v is None else v.to(DEV)) for k, v in synth.make_inputs(wl, 2).items()}
    cfg = binding.config_of(wl)
    outs = []
    for poison in (False, True):
        out = binding.alloc_outputs(cfg, DEV, x_disp=True, y_disp=True)
        ws = binding.alloc_workspace(cfg)
        if poison:
            out.x_disp.fill_(float("nan"))
            out.y_disp.fill_(float("nan"))
            ws.fill_(0xFF)  # NaN bit patterns everywhere in the workspace
        binding.moe_layer_forward(cfg, inp["x"], inp, out, ws)
        torch.cuda.synchronize()
        outs.append(out)
    a, b = outs
    for f in ("y", "expert_ids", "gates", "slots", "load", "kept", "aux_loss", "drop_mask"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    assert torch.isfinite(b.y.float()).all()


@pytest.mark.parametrize("T,d,F", [(400, 256, 384), (400, 1024, 2048), (200, 1024, 2048)])
def test_int8_path_equals_bf16_path_on_power_of_two_scales(T, d, F):
    # same tile shape on both paths -> same MFMA order -> bit-identical outputs
    wl = W("q", T=T, d=d, E=4, k=2, d_ff=F, capacity_factor=1.0, wfmt="int8")
    inp = synth.make_inputs(wl, seed=4, pow2_scales=True)
    deq = {}
    for n in ("w1", "w2"):
        s = inp[n + "_scale"].float().repeat_interleave(128, dim=-1)
        w = inp[n].float() * s
        assert torch.equal(w.to(torch.bfloat16).float(), w)  # exactly bf16
        deq[n] = w.to(torch.bfloat16)
    dinp = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    _, out_q, _ = _run_layer(wl, dinp)
    wl_b = wl.replace(wfmt="plain")
    dinp_b = dict(dinp, w1=deq["w1"].to(DEV), w2=deq["w2"].to(DEV), w1_scale=None, w2_scale=None)
    _, out_b, _ = _run_layer(wl_b, dinp_b)
    assert torch.equal(out_q.y, out_b.y)
    assert torch.equal(out_q.kept, out_b.kept)
    for e, n in enumerate(out_q.kept.tolist()):  # rows past kept[e] are never written
        assert torch.equal(out_q.y_disp[e, :n], out_b.y_disp[e, :n])


def test_dense_overlap_matches_in_order_layer():
    # the dense MLP on the side stream (fork/join) gives the same bits as the
    # dense MLP in order on the caller's stream, over repeated calls
    wl = W("ov", T=700, d=256, E=8, k=2, d_ff=512, capacity_factor=1.0, d_ff_dense=512,
           pr_moe=True, add_skip=True)
    dinp = {k: (None if v is None else v.to(DEV)) for k, v in synth.make_inputs(wl, seed=11).items()}
    _, ref, _ = _run_layer(wl, dinp, overlap_dense=False)
    for _ in range(3):
        _, out, _ = _run_layer(wl, dinp, overlap_dense=True)
        assert torch.equal(out.y, ref.y)
        assert torch.equal(out.dense_out, ref.dense_out)


def test_empty_batch():
    wl = W("empty", T=0, d=64, E=4, k=2, d_ff=64, capacity_factor=1.0)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in synth.make_inputs(wl, 0).items()}
    cfg = binding.config_of(wl)
    assert binding.capacity(cfg) == 0
    out = binding.alloc_outputs(cfg, DEV)
    out.load.fill_(-5)
    out.kept.fill_(-5)
    binding.moe_layer_forward(cfg, inp["x"], inp, out, binding.alloc_workspace(cfg))
    torch.cuda.synchronize()
    assert out.load.tolist() == [0] * 4 and out.kept.tolist() == [0] * 4
    assert float(out.aux_loss.item()) == 0.0


# ------------------------------------------------------------ full-size workloads
# ------------------------------------------------------------ x_disp not kept
# With read_x_rows and without x_disp among the outputs, the first expert
# GEMM reads the token rows of x through the slot -> token table that
# placement writes (token-order dispatch, bf16 activations, shapes on the DMA
# tiles) and no gathered copy is made.  Every output must equal, bit for bit,
# the run that keeps x_disp (checked against the oracle in the tests above),
# and the expert rows are checked against the oracle as well.  Without
# read_x_rows (the default) the gathered buffer goes to the workspace.
ROW_TABLE = [w for w in SMALL if w.act == "bf16"] + [
    # int8 experts on the scheduled 256-row DMA tiles (E >= 32, C > 128, d
    # and d_ff multiples of 1024) and on the 128-row ones (C <= 128)
    W("int8_sched_rows", T=2400, d=1024, E=32, k=2, d_ff=1024, capacity_factor=1.25,
      wfmt="int8", zipf_s=1.2),
    W("int8_rows_c128", T=1000, d=1024, E=16, k=2, d_ff=2048, capacity_factor=1.0,
      wfmt="int8"),
]


def _layer_outputs(wl, inp, keep_x_disp, wfmt=None, read_x_rows=False):
    kw = {"wfmt": wfmt} if wfmt else {}
    cfg = binding.config_of(wl, read_x_rows=read_x_rows, **kw)
    out = binding.alloc_outputs(cfg, DEV, logits=True, x_disp=keep_x_disp, y_disp=True,
                                dense_out=True)
    check_guards = guard_outputs(out)
    binding.moe_layer_forward(cfg, inp["x"], inp, out, binding.alloc_workspace(cfg))
    torch.cuda.synchronize()
    check_guards()
    return out


def _same_layer_outputs(a, b, E):
    for name in ("y", "expert_ids", "gates", "slots", "drop_mask", "load", "kept", "aux_loss",
                 "logits", "dense_out"):
        u, v = getattr(a, name), getattr(b, name)
        assert (u is None) == (v is None), name
        if u is not None:
            assert torch.equal(u, v), name
    kept = a.kept.cpu().tolist()
    for e in range(E):  # rows past kept[e] are not written
        assert torch.equal(a.y_disp[e, :kept[e]], b.y_disp[e, :kept[e]]), f"y_disp[{e}]"


@pytest.mark.parametrize("wl", ROW_TABLE, ids=[w.name for w in ROW_TABLE])
def test_layer_without_x_disp_reads_token_rows(wl):
    print(f"[row_table] {wl.name}", flush=True)
    inp = synth.make_inputs(wl, seed=0, device=DEV)
    a = _layer_outputs(wl, inp, True)
    b = _layer_outputs(wl, inp, False, read_x_rows=True)
    c = _layer_outputs(wl, inp, False)  # gathered into the workspace
    assert b.x_disp is None and c.x_disp is None
    _same_layer_outputs(a, b, wl.E)
    _same_layer_outputs(a, c, wl.E)
    # the first and last kept row of every active expert against the oracle
    inv = _inverse(to_np(b.expert_ids), to_np(b.slots), wl.E)
    want, where = {}, []
    for e in range(wl.E):
        for i in sorted({0, len(inv[e]) - 1}) if inv[e] else ():
            s_, t_, _ = inv[e][i]
            want.setdefault(e, []).append(t_)
            where.append((e, s_))
    rows = oracle_rows_by_expert(inp["x"].cpu(), inp, want)
    ref_rows = np.concatenate([rows[e] for e in sorted(rows)])
    es = torch.as_tensor([w[0] for w in where], device=DEV)
    ss = torch.as_tensor([w[1] for w in where], device=DEV)
    check_close("y_disp (first/last kept row of every expert)", b.y_disp[es, ss], ref_rows,
                TAU["bf16"])


@pytest.mark.parametrize("wl", ROW_TABLE[:2], ids=[w.name for w in ROW_TABLE[:2]])
def test_read_x_rows_falls_back_to_the_gather(wl):
    # gate-priority dispatch has no slot -> token table: read_x_rows then
    # gathers as usual, bit for bit the same outputs
    print(f"[read_x_rows gate priority] {wl.name}", flush=True)
    inp = synth.make_inputs(wl, seed=1, device=DEV)
    outs = []
    for rows_direct in (False, True):
        cfg = binding.config_of(wl, drop_policy="gate_priority", read_x_rows=rows_direct)
        out = binding.alloc_outputs(cfg, DEV, logits=True, y_disp=True, dense_out=True)
        binding.moe_layer_forward(cfg, inp["x"], inp, out, binding.alloc_workspace(cfg))
        torch.cuda.synchronize()
        outs.append(out)
    _same_layer_outputs(outs[0], outs[1], wl.E)


def _inverse(ids, slots, E):
    """per expert: list of (slot, token, j) of its kept assignments, by slot"""
    rows = [[] for _ in range(E)]
    for t, j in zip(*np.nonzero(slots >= 0)):
        rows[ids[t, j]].append((int(slots[t, j]), int(t), int(j)))
    return [sorted(r) for r in rows]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size_layer_sampled(name):
    wl = workloads.WORKLOADS[name]
    print(f"[full_size] {name}", flush=True)
    inp = synth.make_inputs(wl, seed=0, device=DEV)
    cfg, out, m = _run_layer(wl, inp)
    C = binding.capacity(cfg)
    x = inp["x"].cpu()
    b = None if inp["b_router"] is None else inp["b_router"].cpu()
    r = oracle.route(x, inp["w_router"].cpu(), wl.k, bias=b, normalize=wl.normalize_topk)
    loss, _, _ = oracle.aux_loss(r["ids"], r["probs"], wl.aux_alpha)
    dsp = oracle.dispatch(r["ids"], wl.E, oracle.capacity(wl.T, wl.E, wl.k, wl.capacity_factor))
    ref = dict(r, aux=loss, **dsp)
    bad = _check_routing(wl, out, ref, C)
    assert len(bad) == 0, "near-tie flips: sampled expert checks below assume none"
    tau = TAU[wl.act]
    rng = np.random.default_rng(0)
    inv = _inverse(ref["ids"], ref["slots"], wl.E)
    xd = out.x_disp
    # the first and last kept row of every active expert: the gather is an
    # exact copy, the expert rows match the oracle's FFN of those tokens
    want, where = {}, []
    for e in range(wl.E):
        if inv[e]:
            ends = sorted({0, len(inv[e]) - 1})
            for i in ends:
                s_, t_, _ = inv[e][i]
                want.setdefault(e, []).append(t_)
                where.append((e, s_, t_))
    es = torch.as_tensor([w[0] for w in where], device=DEV)
    ss = torch.as_tensor([w[1] for w in where], device=DEV)
    assert torch.equal(xd[es, ss].cpu(), x[[w[2] for w in where]])
    rows = oracle_rows_by_expert(x, inp, want)
    ref_rows = np.concatenate([rows[e] for e in sorted(rows)])
    check_close("y_disp (first/last kept row of every expert)", out.y_disp[es, ss], ref_rows,
                tau)
    print(f"  {len(where)} expert rows over {len(rows)} active experts", flush=True)
    # 64 sampled tokens: every kept expert row of theirs, M, D and y
    toks = np.sort(rng.choice(wl.T, size=min(64, wl.T), replace=False))
    dref = None
    if wl.pr_moe:
        dref = oracle.ffn_rows(x[torch.as_tensor(toks)], inp["wm1"].cpu(), inp["wm2"].cpu())
        check_close("D", out.dense_out[torch.as_tensor(toks, device=DEV)], dref, tau)
    err_m, n_rows = check_expert_terms(wl, x, inp, ref["ids"], ref["slots"], ref["gates"],
                                       out.y_disp, m, out.y, toks, dense=dref)
    print(f"  {len(toks)} tokens, {n_rows} of their rows kept; M rel err {err_m:.2e}",
          flush=True)
    if wl.act == "bf16":
        # as the benchmark runs it: x_disp not kept (gathered into the
        # workspace) and bf16 expert weights packed, and the same with the
        # first expert GEMM reading the token rows through the slot -> token
        # table (read_x_rows): every output equal to this run's
        wts = inp
        wfmt = "packed" if wl.wfmt == "plain" and wl.d % 128 == 0 and wl.d_ff % 128 == 0 else None
        if wfmt:
            cfgp = binding.config_of(wl, wfmt=wfmt)
            wts = dict(inp, w1=binding.pack_expert_weights(cfgp, 1, inp["w1"]),
                       w2=binding.pack_expert_weights(cfgp, 2, inp["w2"]))
        for rows_direct in (False, True):
            b = _layer_outputs(wl, wts, False, wfmt=wfmt, read_x_rows=rows_direct)
            _same_layer_outputs(out, b, wl.E)
            del b
            print(f"  without x_disp{' (packed weights)' if wfmt else ''}"
                  f"{', read_x_rows' if rows_direct else ''}: outputs identical", flush=True)
        del wts
    del inp, out, m
    torch.cuda.empty_cache()
