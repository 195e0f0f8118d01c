"""Benchmark: MoE-layer forward tokens/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--headline-only]
                    [--no-cpu-baseline] [--copy-calibration GIB]
                    [--backward | --train] [--recompute]
    python bench.py --pmc-summary FETCH.csv WRITE.csv --label L --symbol RE
                    --workload NAME --copy-gib G --command "..."   (no GPU)

A step is one moe_layer_forward (router + softmax/top-k + aux loss, dispatch,
PR-MoE dense MLP, expert FFNs, combine) over one batch of seeded synthetic
tokens already resident in HBM (--backward: one moe_layer_backward of that
forward; --train: forward keeping the FFN activations, then the backward).
The default workload is the 1.3B+PR-MoE-128
layer (T=16384, d=2048, E=128 top-1 experts with d_ff=8192 plus a dense MLP
with d_ff=8192, bf16); its record is the top level of the JSON line.  Without
--workload (and without a variant flag) the other four workloads -- the tiny
fp32 layer, the 350M+MoE-128 layer, the decode layer and the skewed int8
layer -- are measured the same way and reported under "workloads" (their own
records, not part of "value").  One JSON line is printed:

  value      whole-job tokens/s over the K timed steps (host clock around
             device-synchronised steps)
  roofline   the dominant kernel (most time per step in a two-step survey
             after the warmup, where every kernel is timed): algorithmic bytes
             or FLOPs per launch divided by its mean launch time, measured
             with HIP events recorded on the launch stream around that
             kernel's launches during the timed steps (no other kernel carries
             events there); traffic = HBM bytes per launch from the committed
             rocprofv3 counter summary when it was taken on the current kernel
             source, else null
  layer      the whole layer's algorithmic FLOPs and HBM bytes per step
             (hidden rows excluded) against the bf16 MFMA and HBM peaks
  routing    assignments, drops, expert load and kept extremes, near-tie
             tokens (k-th and (k+1)-th fp32 logits within 1e-5) and whether
             the expert ids equal the oracle's on every other token
  kernels    per-kernel mean launch times from the survey steps
  isolated   (PR-MoE with the dense MLP overlapped) every kernel's time in
             two more survey steps with the dense MLP run in order, and its
             rate against the roofline; the overlapped step's kernels share
             the chip, so their spans in `kernels` include each other's time
  cold_cache steps timed one by one after a 512 MiB read that evicts the
             Infinity Cache (the timed steps above run back to back, so inputs
             smaller than the cache may be partly warm there)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
             (routing and dispatch on every token, expert FFN and dense MLP on a
             seeded token sample, extrapolated linearly in tokens)

--copy-calibration G copies a G GiB device buffer three times before the
warmup, so that a rocprofv3 --pmc run of the same command also counts a plain
copy of known size.  --pmc-summary turns the counter_collection.csv files of
a FETCH_SIZE run and a WRITE_SIZE run into profiles/<label>__<workload>__pmc.txt:
HBM bytes per launch of the kernel whose symbol matches RE, scaled by
(known copy bytes / counted copy bytes) of the calibration copy.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1.3B+MoE-128 shape; % bf16 MFMA peak / % HBM BW"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector/matrix, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample (headline workload)")
    p.add_argument("--sub-cpu-seconds", type=float, default=6.0,
                   help="target CPU time of the oracle sample of each other workload")
    p.add_argument("--headline-only", action="store_true",
                   help="skip the sub-records of the other four workloads")
    p.add_argument("--drop-policy", default="token_order", choices=["token_order", "gate_priority"])
    p.add_argument("--z-loss", action="store_true", help="also compute the router z-loss")
    p.add_argument("--backward", action="store_true",
                   help="time the layer backward (after one forward) instead of the forward")
    p.add_argument("--train", action="store_true",
                   help="time forward (keeping the FFN activations) + backward as one step")
    p.add_argument("--router", default="topk", choices=["topk", "top_p", "cosine", "noisy_topk"],
                   help="router variant (the workloads use topk)")
    p.add_argument("--top-p", type=float, default=0.5, help="top_p router: threshold P")
    p.add_argument("--cos-tau", type=float, default=0.1, help="cosine router: temperature")
    p.add_argument("--cos-dim", type=int, default=64, help="cosine router: projection width")
    p.add_argument("--k", type=int, default=0, help="override the workload's k (slots per token)")
    p.add_argument("--router-losses", action="store_true",
                   help="also compute the Importance and Load losses (weights 0.01)")
    p.add_argument("--recompute", action="store_true",
                   help="backward / train: do not keep the FFN activations in the forward; "
                        "the backward recomputes them")
    p.add_argument("--serial", action="store_true",
                   help="PR-MoE: dense MLP in order on the launch stream (no side-stream overlap)")
    p.add_argument("--read-x-rows", action="store_true",
                   help="the first expert GEMM reads the token rows of x through the slot -> "
                        "token table instead of the gathered [E, C, d] buffer (default: gather)")
    p.add_argument("--expert-weights", default="auto", choices=["auto", "plain", "packed"],
                   help="bf16 expert weights row-major (plain) or in 128-row x 64-k blocks "
                        "(packed once before timing); auto = packed for a forward pass "
                        "with bf16 experts and d, d_ff multiples of 128")
    p.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB")
    p.add_argument("--cold-steps", type=int, default=5,
                   help="extra steps, each after a 512 MiB read that evicts the 256 MB "
                        "Infinity Cache, timed one by one with HIP events (0 = skip)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    p.add_argument("--stats-summary", metavar="CSV",
                   help="kernel_stats.csv of a rocprofv3 --kernel-trace --stats run: write "
                        "profiles/<label>__<workload>__kernel_stats.txt")
    p.add_argument("--sq-summary", nargs="+", metavar="CSV",
                   help="counter_collection.csv files of SQ/GRBM counter runs: write "
                        "profiles/<label>__<workload>__sq_counters.txt")
    p.add_argument("--label")
    p.add_argument("--symbol")
    p.add_argument("--copy-gib", type=float, default=1.0)
    p.add_argument("--command", default="")
    return p.parse_args()


# ------------------------------------------------------------- algorithmic work
def kernel_work(wl, kept, cfg_C, router="topk", cos_dim=64):
    """Algorithmic bytes and FLOPs of one launch of each kernel class.

    Expert GEMM1: reads the weights of experts with >= 1 kept row once and
    the kept rows of x_disp; FLOPs 2*N_kept*d*d_ff.  Expert GEMM2: weights of
    active experts, kept rows of y_disp out; FLOPs 2*N_kept*d_ff*d.  The
    hidden rows H are excluded (they can stay on chip; this build writes and
    reads them, reported as h_bytes).  Dense GEMM1/2: x, Wm1, Hd / Hd, Wm2,
    D; FLOPs 2*T*d*d_ff_dense each.  int8 weights count 1 byte plus 2 bytes
    of scale per 128.
    """
    sa = 4 if wl.act == "f32" else 2
    n_kept = int(sum(kept))
    n_act = int(sum(1 for v in kept if v > 0))
    if wl.wfmt == "int8":
        wbytes = n_act * wl.d * wl.d_ff * (1 + 2 / 128)
    else:
        wbytes = n_act * wl.d * wl.d_ff * sa
    # the hidden rows H (written by GEMM1, read by GEMM2) are not counted:
    # the method need not send them to HBM; h_bytes reports them apart
    h = n_kept * wl.d_ff * sa
    out = {
        "expert_gemm1": dict(bytes=wbytes + n_kept * wl.d * sa,
                             flops=2.0 * n_kept * wl.d * wl.d_ff, h_bytes=h),
        "expert_gemm2": dict(bytes=wbytes + n_kept * wl.d * sa,
                             flops=2.0 * n_kept * wl.d_ff * wl.d, h_bytes=h),
    }
    if wl.pr_moe:
        T, d, F = wl.T, wl.d, wl.d_ff_dense
        out["dense_gemm1"] = dict(bytes=(T * d + F * d + T * F) * sa, flops=2.0 * T * d * F)
        out["dense_gemm2"] = dict(bytes=(T * F + d * F + T * d) * sa, flops=2.0 * T * d * F)
    out["router"] = dict(bytes=(wl.T * wl.d + wl.E * wl.d) * sa + wl.T * wl.k * 8,
                         flops=2.0 * wl.T * wl.d * wl.E)
    # backward GEMMs (bwd_*): the expert products over the kept rows read the
    # active experts' weights (dZ, dX) or write their gradients (dW1, dW2)
    K = n_kept
    out["bwd_expert_z"] = dict(bytes=wbytes + K * (wl.d + wl.d_ff) * sa,
                               flops=2.0 * K * wl.d * wl.d_ff)
    out["bwd_expert_dz"] = dict(bytes=wbytes + K * (wl.d + 2 * wl.d_ff) * sa,
                                flops=2.0 * K * wl.d * wl.d_ff)
    out["bwd_expert_dx"] = dict(bytes=wbytes + K * (wl.d_ff + wl.d) * sa,
                                flops=2.0 * K * wl.d * wl.d_ff)
    out["bwd_expert_dw"] = dict(bytes=wl.E * wl.d * wl.d_ff * sa + K * (wl.d + wl.d_ff) * sa,
                                flops=2.0 * K * wl.d * wl.d_ff)
    if wl.pr_moe:
        T, d, F = wl.T, wl.d, wl.d_ff_dense
        for c in ("bwd_dense_z", "bwd_dense_dz", "bwd_dense_dx", "bwd_dense_dw"):
            out[c] = dict(bytes=(T * d + F * d + T * F) * sa, flops=2.0 * T * d * F)
    out["bwd_router"] = dict(bytes=(wl.T * wl.d + wl.E * wl.d + wl.T * wl.E) * sa,
                             flops=2.0 * wl.T * wl.d * wl.E)
    # router variants: raw products into [T, ns] fp32 (ns = E, 2E or the
    # cosine width), the cosine logits, the variant epilogue
    ns = {"noisy_topk": 2 * wl.E, "cosine": cos_dim}.get(router, wl.E)
    out["router_scores"] = dict(bytes=(wl.T * wl.d + ns * wl.d) * sa + wl.T * ns * 4,
                                flops=2.0 * wl.T * wl.d * ns)
    out["cosine_logits"] = dict(bytes=(wl.T * cos_dim + wl.E * cos_dim + wl.T * wl.E) * 4,
                                flops=2.0 * wl.T * wl.E * cos_dim)
    out["route_logits"] = dict(bytes=wl.T * ns * 4 + (wl.T * wl.E * 4 if router == "noisy_topk"
                                                      else 0) + wl.T * wl.k * 8,
                               flops=0.0)
    out["gather"] = dict(bytes=2.0 * n_kept * wl.d * sa, flops=0.0)
    out["combine"] = dict(bytes=(n_kept + wl.T * (1 + int(wl.add_skip) + int(wl.pr_moe)))
                          * wl.d * sa, flops=2.0 * n_kept * wl.d)
    return out


def layer_work(wl, kept):
    """Algorithmic FLOPs and HBM bytes of one whole layer call: the router
    reads x once and W_r; the active experts' weights are read once (int8: 1
    byte + 2 bytes of scale per 128); the gather reads and writes the kept
    rows; the expert GEMMs read x_disp and write y_disp; the combine reads the
    kept expert rows and the base terms and writes y; PR-MoE adds its dense
    weights and D; ids/gates/slots/drop mask are written once.  The hidden
    rows of the experts and of the dense MLP are excluded."""
    sa = 4 if wl.act == "f32" else 2
    n_kept = int(sum(kept))
    n_act = int(sum(1 for v in kept if v > 0))
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.d_ff
    sw = (1 + 2 / 128) if wl.wfmt == "int8" else sa
    flops = 2.0 * T * d * E + 4.0 * n_kept * d * F + 2.0 * n_kept * d
    byt = (sa * T * d + sa * E * d + sw * n_act * 2 * d * F + 2 * sa * n_kept * d
           + 2 * sa * n_kept * d + sa * (n_kept + T * (1 + int(wl.add_skip) + int(wl.pr_moe))) * d
           + T * k * (4 + 4 + 4 + 1))
    if wl.pr_moe:
        flops += 4.0 * T * d * wl.d_ff_dense
        byt += sa * 2 * d * wl.d_ff_dense + sa * T * d
    return flops, byt


def classify(name: str) -> str | None:
    """Work class of a library kernel name (names are "<role>:<tile>" for
    GEMMs, the kernel's own name otherwise)."""
    for prefix, cls in (("expert_ffn1", "expert_gemm1"), ("expert_ffn2", "expert_gemm2"),
                        ("dense_mlp1", "dense_gemm1"), ("dense_mlp2", "dense_gemm2"),
                        ("bwd_expert_z", "bwd_expert_z"), ("bwd_expert_dz", "bwd_expert_dz"),
                        ("bwd_expert_dx", "bwd_expert_dx"), ("bwd_expert_dw", "bwd_expert_dw"),
                        ("bwd_dense_z", "bwd_dense_z"), ("bwd_dense_dz", "bwd_dense_dz"),
                        ("bwd_dense_dx", "bwd_dense_dx"), ("bwd_dense_dw", "bwd_dense_dw"),
                        ("bwd_router_", "bwd_router"), ("router_scores", "router_scores"),
                        ("cosine_logits", "cosine_logits"), ("route_logits", "route_logits"),
                        ("router", "router"), ("gather", "gather"), ("combine", "combine")):
        if name.startswith(prefix):
            return cls
    return None


def src_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "mixture_experts_layer_24_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/<kernel>__<workload>__pmc.txt if its
    recorded source hash matches the current kernels, else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel.replace(':', '_')}__{workload}__pmc.txt")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m = re.search(r"source_hash:\s*(\w+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != src_hash():
        return None
    return float(b.group(1))


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, inp, target_s):
    import numpy as np
    import torch

    import oracle
    t0 = time.perf_counter()
    x = inp["x"].cpu()
    b = None if inp["b_router"] is None else inp["b_router"].cpu()
    r = oracle.route(x, inp["w_router"].cpu(), wl.k, bias=b, normalize=wl.normalize_topk)
    oracle.aux_loss(r["ids"], r["probs"], wl.aux_alpha)
    C = oracle.capacity(wl.T, wl.E, wl.k, wl.capacity_factor)
    dsp = oracle.dispatch(r["ids"], wl.E, C)
    t_route = time.perf_counter() - t0

    rng = np.random.default_rng(1234)
    order = rng.permutation(wl.T)
    w_cache = {}

    def ffn_tokens(toks):
        """expert FFN + dense MLP + combine for the given tokens; returns seconds"""
        need = {}
        for t in toks:
            for j in range(wl.k):
                if dsp["slots"][t, j] >= 0:
                    need.setdefault(int(r["ids"][t, j]), []).append(int(t))
        # weights are copied to host outside the timed part
        for e in need:
            if e not in w_cache:
                s1 = None if inp["w1_scale"] is None else inp["w1_scale"][e].cpu()
                s2 = None if inp["w2_scale"] is None else inp["w2_scale"][e].cpu()
                w_cache[e] = (inp["w1"][e].cpu(), inp["w2"][e].cpu(), s1, s2)
        dense_w = (inp["wm1"].cpu(), inp["wm2"].cpu()) if wl.pr_moe else None
        t1 = time.perf_counter()
        for e, ts in need.items():
            w1, w2, s1, s2 = w_cache[e]
            oracle.ffn_rows(x[ts], w1, w2, s1, s2)
        if dense_w is not None:
            oracle.ffn_rows(x[list(toks)], *dense_w)
        return time.perf_counter() - t1

    # grow the sample in rounds sized from the rate measured so far, until it
    # has used about the time budget (small rounds parallelise worse, so the
    # first estimate is low)
    budget = max(target_s - t_route, 1.0)
    n, t_ffn = 0, 0.0
    step = 64
    while n < wl.T and t_ffn < 0.8 * budget:
        m = int(min(wl.T - n, max(16, step)))
        t_ffn += ffn_tokens(order[n:n + m])
        n += m
        rate = t_ffn / n
        step = (budget - t_ffn) / max(rate, 1e-9)
    t_total = t_route + t_ffn * (wl.T / n)
    rec = {
        "value": wl.T / t_total, "unit": "tokens/s", "cores": oracle.threads(),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"fp64 oracle: routing, aux loss and dispatch on all {wl.T} tokens "
                   f"({t_route:.2f} s); expert FFN{' + dense MLP' if wl.pr_moe else ''} "
                   f"on a seeded sample of {n} tokens ({t_ffn:.2f} s)" +
                   (f", extrapolated linearly to {wl.T} tokens" if n < wl.T else
                    " (every token)")),
    }
    return rec, r


# ------------------------------------------------------------- main
def pmc_rows(path):
    """(kernel name, counter value) per dispatch from a rocprofv3
    counter_collection.csv (counter values of one dispatch summed)."""
    import csv
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            nm = r["Kernel_Name"]
            v = float(r["Counter_Value"])
            if key in per:
                per[key] = (nm, per[key][1] + v)
            else:
                per[key] = (nm, v)
    return list(per.values())


def pmc_summary(args):
    """Write profiles/<label>__<workload>__pmc.txt from a FETCH_SIZE and a
    WRITE_SIZE counter run (values in KiB per dispatch)."""
    known = args.copy_gib * (1 << 30)
    out = {}
    for ctr, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.pmc_summary):
        rows = pmc_rows(path)
        # the calibration copies: copy kernels whose count is within a factor of
        # four of the known size (the other copies are input uploads of <= 64 MiB)
        cal = [v * 1024.0 for n, v in rows if "copy" in n.lower() and v * 1024.0 > 0.25 * known]
        if not cal:
            raise SystemExit(f"{path}: no calibration copy of ~{known:.0f} bytes found")
        factor = known / (sum(cal) / len(cal))
        mine = [v * 1024.0 for n, v in rows if re.search(args.symbol, n)]
        if not mine:
            raise SystemExit(f"{path}: no dispatch of a kernel matching {args.symbol!r}")
        raw = sum(mine) / len(mine)
        out[ctr] = (raw, factor, len(mine), len(cal))
    hbm = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][1] + out["WRITE_SIZE"][0] * out["WRITE_SIZE"][1]
    lines = [f"# rocprofv3 HBM traffic -- kernel {args.label}, workload {args.workload}",
             f"# command: {args.command}",
             "# ($REPO is the repository root)",
             f"source_hash: {src_hash()}",
             f"symbol_regex: {args.symbol}"]
    for ctr, (raw, factor, n, ncal) in out.items():
        lines.append(f"{ctr}: {raw:.6e} bytes per dispatch counted (mean of {n} dispatches); "
                     f"calibration copy of {known:.0f} bytes counted {known / factor:.6e} "
                     f"({ncal} copies) -> scale {factor:.4f}")
    lines.append(f"hbm_bytes_per_launch: {hbm:.6e}")
    dst = os.path.join(ROOT, "profiles",
                       f"{args.label.replace(':', '_')}__{args.workload}__pmc.txt")
    open(dst, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def routing_record(wl, out, C, ref_route=None):
    """Expert load, drops and near-ties of the measured call.  Near-ties are
    tokens whose k-th and (k+1)-th fp32 router logits lie within 1e-5 (the
    oracle's fp64 logits rounded to fp32 when the oracle routed every token,
    else the layer's own fp32 logits); with the oracle's routing the layer's
    expert ids are also compared on every other token."""
    import numpy as np
    load = out.load.cpu().numpy()
    kept = out.kept.cpu().numpy()
    ids = out.expert_ids.cpu().numpy()
    assigned = int((ids >= 0).sum())
    n_kept = int(kept.sum())
    rec = {"assignments": assigned, "kept": n_kept, "dropped": assigned - n_kept,
           "drop_rate": round((assigned - n_kept) / max(assigned, 1), 5), "capacity": C,
           "load_min": int(load.min()), "load_max": int(load.max()),
           "kept_min": int(kept.min()), "kept_max": int(kept.max()),
           "active_experts": int((kept > 0).sum())}
    logits = None
    if ref_route is not None:
        logits = np.asarray(ref_route["logits"], np.float64).astype(np.float32)
        src = "oracle fp64 logits rounded to fp32"
    elif out.logits is not None:
        logits = out.logits.cpu().numpy()
        src = "layer fp32 logits"
    if logits is not None and wl.k < wl.E:
        srt = -np.sort(-logits.astype(np.float64), axis=1)
        near = np.nonzero(srt[:, wl.k - 1] - srt[:, wl.k] < 1e-5)[0]
        rec["near_ties"] = int(len(near))
        rec["near_tie_tokens"] = near[:16].tolist()
        rec["near_tie_source"] = src
        if ref_route is not None:
            bad = np.nonzero((ids != ref_route["ids"]).any(axis=1))[0]
            rec["ids_equal_oracle_except_near_ties"] = bool(set(bad.tolist()) <= set(near.tolist()))
            rec["ids_differing"] = int(len(bad))
    return rec


def run_workload(name, args, headline=True):
    """Time one workload; returns its JSON record."""
    import torch

    from mixture_experts_layer_24_amd import binding, synth, workloads

    wl = workloads.WORKLOADS[name]
    if args.k:
        wl = wl.replace(k=args.k)
    dev = "cuda:0"
    steps = args.steps if headline else max(args.steps, args.sub_steps.get(name, args.steps))
    inp = synth.make_inputs(wl, seed=args.seed, device=dev)
    rkw = {}
    if args.router != "topk" or args.router_losses:
        inp.update(synth.router_inputs(wl, args.router, seed=args.seed, device=dev,
                                       cos_dim=args.cos_dim))
        rkw = dict(router=args.router)
        if args.router == "top_p":
            rkw["top_p"] = args.top_p
        if args.router == "cosine":
            rkw.update(cos_tau=args.cos_tau, cos_dim=args.cos_dim)
        if args.router_losses:
            rkw.update(w_importance=0.01, w_load=0.01)
    bwd = args.backward or args.train
    packable = (wl.act == "bf16" and wl.wfmt == "plain" and wl.d % 128 == 0 and
                wl.d_ff % 128 == 0)
    packed = (args.expert_weights == "packed" and packable) or (
        args.expert_weights == "auto" and packable and not bwd)
    if args.expert_weights == "packed" and (not packable or bwd) and headline:
        raise SystemExit("bench.py: packed expert weights need a forward pass with bf16 "
                         "experts and d, d_ff multiples of 128")
    if packed:
        wl = wl.replace(wfmt="packed")
    cfg = binding.config_of(wl, overlap_dense=not args.serial, drop_policy=args.drop_policy,
                            read_x_rows=args.read_x_rows, **rkw)
    oracle_inp = inp  # the CPU oracle reads the row-major weights
    if packed:  # once, where a model's weights are loaded: outside the timed steps
        inp = dict(inp, w1=binding.pack_expert_weights(cfg, 1, inp["w1"]),
                   w2=binding.pack_expert_weights(cfg, 2, inp["w2"]))
        torch.cuda.synchronize()
    C = binding.capacity(cfg)
    out = binding.alloc_outputs(cfg, dev, z_loss=args.z_loss, logits=bwd, x_disp=bwd,
                                y_disp=bwd, saved_activations=bwd and not args.recompute,
                                importance_loss=args.router_losses,
                                load_loss=args.router_losses)
    ws = binding.alloc_workspace(cfg, device=dev)
    stream = torch.cuda.current_stream()

    def forward():
        binding.moe_layer_forward(cfg, inp["x"], inp, out, ws, stream)

    step = forward
    if bwd:
        forward()  # the forward whose outputs the backward reads
        dy = synth.normal((wl.T, wl.d), 1.0, args.seed + 1, "dy", dev, torch.bfloat16)
        grads = binding.alloc_grads(cfg, dev)
        ws_b = binding.alloc_workspace(cfg, binding.ENTRY_BACKWARD, device=dev)

        def backward():
            binding.moe_layer_backward(cfg, inp["x"], inp, out, dy, grads, ws_b, g_aux=0.01,
                                       g_z=0.001, stream=stream)

        def train_step():
            forward()
            backward()

        step = train_step if args.train else backward

    if args.copy_calibration > 0 and headline:
        n = int(args.copy_calibration * (1 << 30))
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copies of {n} bytes done", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {name}: warmup {args.warmup} done", file=sys.stderr, flush=True)

    # survey: two steps with a HIP event pair around every kernel, for the
    # per-kernel table and to find the dominant kernel (most time per step)
    survey_steps = 2
    binding.profile_reset()
    binding.profile_filter(None)
    binding.profile_enable(True)
    for _ in range(survey_steps):
        step()
    torch.cuda.synchronize()
    binding.profile_enable(False)
    survey = binding.profile_read()
    dom_name = max(survey, key=lambda n: survey[n][1])

    # timed region: host clock around K device-synchronised steps; the library
    # records a HIP event pair on the launch stream around the dominant
    # kernel's launches only (an event pair around every kernel would add a
    # bubble per launch to the steps being timed)
    binding.profile_reset()
    binding.profile_filter(dom_name)
    binding.profile_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    binding.profile_enable(False)
    binding.profile_filter(None)
    prof = binding.profile_read()
    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / steps
    ev_ms = ev0.elapsed_time(ev1) / steps
    print(f"[bench] {name}: {steps} steps: {ms_per_step:.3f} ms/step (events {ev_ms:.3f})",
          file=sys.stderr, flush=True)

    # cold-cache steps: the timed steps above run back to back, so inputs
    # smaller than the Infinity Cache (the token batch, the router weights)
    # can be partly resident from the previous step; here each step follows a
    # 512 MiB read and is timed alone (the read is outside the event pair)
    cold = None
    if args.cold_steps > 0:
        flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        times = []
        for i in range(args.cold_steps):
            # a 512 MiB read: evicts without leaving dirty lines to drain
            # during the timed step
            _ = flush.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        del flush
        times.sort()
        cold = {"ms_per_step_median": round(times[len(times) // 2], 4),
                "ms_per_step_min": round(times[0], 4), "steps": args.cold_steps,
                "evict_read_bytes": 512 << 20}
        print(f"[bench] {name}: cold-cache steps: median {cold['ms_per_step_median']:.3f} ms",
              file=sys.stderr, flush=True)

    # PR-MoE overlapped: the dense MLP's tiles share the chip with the expert
    # path, so the kernels' spans in the survey above include each other's
    # time; two more survey steps with the dense MLP in order give every
    # kernel's time alone (reported as `isolated`, not part of `value`)
    isolated = None
    if wl.pr_moe and not args.serial and not bwd:
        cfg_s = binding.config_of(wl, overlap_dense=False, drop_policy=args.drop_policy,
                                  read_x_rows=args.read_x_rows, **rkw)
        binding.profile_reset()
        binding.profile_filter(None)
        binding.profile_enable(True)
        for _ in range(survey_steps):
            binding.moe_layer_forward(cfg_s, inp["x"], inp, out, ws, stream)
        torch.cuda.synchronize()
        binding.profile_enable(False)
        isolated = {n: tot / cnt for n, (cnt, tot) in binding.profile_read().items()}

    kept = out.kept.cpu().tolist()
    work = kernel_work(wl, kept, C, args.router, args.cos_dim)
    kern = {}
    for n, (cnt, tot) in survey.items():
        kern[n] = {"launches": cnt, "avg_ms": tot / cnt, "ms_per_step": tot / survey_steps,
                   "class": classify(n)}
    cnt, tot = prof[dom_name]
    dom = {"avg_ms": tot / cnt, "class": classify(dom_name)}
    cls = dom["class"]
    wk = work.get(cls, {"bytes": 0.0, "flops": 0.0})
    avg_s = dom["avg_ms"] / 1e3
    ai = wk["flops"] / max(wk["bytes"], 1.0)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma_bound = wl.act == "bf16" and ai > ridge
    if mfma_bound:
        achieved = wk["flops"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = wk["bytes"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = committed_traffic(dom_name, name)
    roof["kernel"] = dom_name
    roof["kernel_class"] = cls
    roof["avg_launch_ms"] = round(dom["avg_ms"], 4)
    roof["algorithmic_bytes"] = wk["bytes"]
    roof["algorithmic_flops"] = wk["flops"]
    if "h_bytes" in wk:
        roof["h_bytes_excluded"] = wk["h_bytes"]
    # the whole layer against both peaks (forward only)
    layer = None
    if not bwd:
        lf, lb = layer_work(wl, kept)
        t_s = ms_per_step / 1e3
        layer = {"algorithmic_flops": lf, "algorithmic_bytes": lb,
                 "tflops": round(lf / t_s / 1e12, 2), "gbs": round(lb / t_s / 1e9, 1),
                 "mfma_frac": round(lf / t_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "hbm_frac": round(lb / t_s / 1e9 / PEAK_HBM_GBS, 4),
                 "floor_ms": round(1e3 * max(lb / (PEAK_HBM_GBS * 1e9),
                                             lf / (PEAK_BF16_TFLOPS * 1e12)), 4),
                 "bound": "hbm" if lf / lb < ridge else "mfma",
                 "excluded": "expert and dense hidden rows (H)"}

    iso = None
    if isolated is not None:
        iso = {"note": "kernels timed with the dense MLP in order (not overlapped); "
                       "not part of value", "kernels": {}}
        for n, ms in sorted(isolated.items(), key=lambda kv: -kv[1]):
            c = classify(n)
            ent = {"avg_ms": round(ms, 4), "class": c}
            w = work.get(c)
            if w and ms > 0:
                if w["flops"] / max(w["bytes"], 1.0) > ridge:
                    ent["tflops"] = round(w["flops"] / (ms / 1e3) / 1e12, 1)
                    ent["mfma_frac"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
                else:
                    ent["gbs"] = round(w["bytes"] / (ms / 1e3) / 1e9, 1)
                    ent["hbm_frac"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
            iso["kernels"][n] = ent

    res = {
        "metric": ("MoE-layer training (forward + backward) tokens/s" if args.train else
                   "MoE-layer backward tokens/s" if args.backward else METRIC),
        "value": round(wl.T * steps / elapsed, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.act == "bf16" else "f32",
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,0.02^2), bf16 RNE)",
        "config": {"workload": name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k,
                   "d_ff": wl.d_ff, "d_ff_dense": wl.d_ff_dense, "capacity": C,
                   "capacity_factor": wl.capacity_factor,
                   "expert_weights": ("bf16 packed (128-row x 64-k blocks, packed once "
                                      "before timing)" if packed else
                                      "int8 + fp16 scale per 128" if wl.wfmt == "int8"
                                      else wl.act + " row-major"),
                   "pr_moe": wl.pr_moe, "add_skip": wl.add_skip,
                   "dense_mlp_overlapped": bool(wl.pr_moe and not args.serial),
                   "x_rows": ("read through the slot -> token table" if args.read_x_rows
                              else "gathered into [E, C, d]"),
                   "drop_policy": args.drop_policy, "z_loss": bool(args.z_loss),
                   "pass": "train" if args.train else "backward" if args.backward else "forward",
                   **({"ffn_activations": "recomputed" if args.recompute else "saved"}
                      if bwd else {}),
                   **({"router": args.router,
                       **{n: v for n, v in rkw.items() if n != "router"}} if rkw else {}),
                   "n_kept": int(sum(kept)), "active_experts": int(sum(v > 0 for v in kept))},
        "roofline": roof,
        "layer": layer,
        "kernels": {n: {"avg_ms": round(k["avg_ms"], 4), "launches_per_step":
                        k["launches"] // survey_steps, "class": k["class"]}
                    for n, k in sorted(kern.items(), key=lambda kv: -kv[1]["ms_per_step"])},
        "cold_cache": cold,
        "isolated": iso,
        "cpu_baseline": None,
    }
    ref_route = None
    if not args.no_cpu_baseline and not bwd and not rkw and not args.k:
        print(f"[bench] {name}: timing the CPU oracle on a bounded sample", file=sys.stderr,
              flush=True)
        budget = args.cpu_seconds if headline else args.sub_cpu_seconds
        res["cpu_baseline"], ref_route = cpu_baseline(wl, oracle_inp, budget)
    if not bwd:
        if ref_route is None and not rkw:  # the layer's own logits for the near-tie count
            out.logits = torch.empty(wl.T, wl.E, dtype=torch.float32, device=dev)
            forward()
            torch.cuda.synchronize()
        res["routing"] = routing_record(wl, out, C, ref_route)
    del inp, oracle_inp, out, ws
    torch.cuda.empty_cache()
    return res


SUB_WORKLOADS = ("tiny_f32", "moe128_350m", "decode_top2", "skewed_top2_int8")


def stats_summary(args):
    """Per-kernel calls, average / min / max duration and share of the traced
    GPU time from a rocprofv3 kernel_stats.csv; torch's own kernels (input
    generation and copies) are named generically."""
    import csv
    rows = []
    with open(args.stats_summary) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), float(r["Percentage"]), r["Name"]))
    rows.sort(key=lambda t: -t[4])
    # median launch duration from the per-launch trace beside the stats file
    # (robust to the few launches of another kind in the run, e.g. the
    # overlapped layer's isolated survey steps)
    med = {}
    trace = os.path.join(os.path.dirname(args.stats_summary),
                         os.path.basename(args.stats_summary).replace("kernel_stats", "kernel_trace"))
    if os.path.exists(trace):
        per = {}
        with open(trace) as fh:
            for r in csv.DictReader(fh):
                per.setdefault(r["Kernel_Name"], []).append(
                    float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
        for n, v in per.items():
            v.sort()
            med[n] = v[len(v) // 2]
    lines = [f"# rocprofv3 kernel statistics -- {args.label}, workload {args.workload}",
             f"# command: {args.command}",
             "# ($REPO is the repository root)",
             f"source_hash: {src_hash()}",
             "# columns: calls, average ns, median ns, min ns, max ns, share of traced GPU time, "
             "kernel", ""]
    for calls, avg, mn, mx, pct, name in rows:
        md = med.get(name, float("nan"))
        if name.startswith("void at::") or name.startswith("at::"):
            name = name.split("<")[0] + "<...> (torch input generation / copies)"
        lines.append(f"{calls:6d} {avg:12.0f} {md:12.0f} {mn:12.0f} {mx:12.0f} {pct:6.2f}%  "
                     f"{name[:160]}")
    dst = os.path.join(ROOT, "profiles", f"{args.label}__{args.workload}__kernel_stats.txt")
    open(dst, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[:12]))


def sq_summary(args):
    """Mean counter values per dispatch of the kernel matching --symbol over
    SQ/GRBM counter runs, and the derived MFMA-busy share, cycles per MFMA,
    LDS-wait share and bank conflicts."""
    import csv
    vals = {}
    for path in args.sq_summary:
        per = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if not re.search(args.symbol, r["Kernel_Name"]):
                    continue
                key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, c), v in per.items():
            vals.setdefault(c, []).append(v)
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {args.symbol!r}")
    mean = {c: sum(v) / len(v) for c, v in vals.items()}
    lines = [f"# rocprofv3 SQ counters -- kernel {args.label}, workload {args.workload}",
             f"# command: {args.command}",
             "# ($REPO is the repository root)",
             f"source_hash: {src_hash()}",
             f"symbol_regex: {args.symbol}",
             "# mean per dispatch, summed over the chip as rocprofv3 reports them"]
    lines += [f"{c}: {mean[c]:.4e} (dispatches {len(vals[c])})" for c in sorted(mean)]
    d = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs share them
        d.append(f"mfma_busy_share: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * mean['GRBM_GUI_ACTIVE'] / 8):.3f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean.get("SQ_INSTS_MFMA"):
        d.append(f"cycles_per_mfma: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / mean['SQ_INSTS_MFMA']:.1f}")
    if "SQ_WAIT_INST_LDS" in mean and mean.get("SQ_BUSY_CYCLES"):
        d.append(f"wait_inst_lds_per_busy_cycle: {mean['SQ_WAIT_INST_LDS'] / mean['SQ_BUSY_CYCLES']:.3f}")
    if "SQ_ACTIVE_INST_VALU" in mean and mean.get("SQ_ACTIVE_INST_ANY"):
        d.append(f"valu_share_of_active_inst: {mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_ACTIVE_INST_ANY']:.3f}")
    if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_ACTIVE_INST_LDS"):
        d.append(f"lds_bank_conflict_per_lds_active: {mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_ACTIVE_INST_LDS']:.3f}")
    lines += ["derived:"] + ["  " + x for x in d]
    dst = os.path.join(ROOT, "profiles",
                       f"{args.label.replace(':', '_')}__{args.workload}__sq_counters.txt")
    open(dst, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.pmc_summary:
        return pmc_summary(args)
    if args.sq_summary:
        return sq_summary(args)
    if args.stats_summary:
        return stats_summary(args)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the expert-parallel all-to-all across GPUs is not part of it)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_layer_24_amd import workloads

    torch.cuda.set_device(0)
    # launch-latency-bound workloads get more timed steps in their sub-records
    args.sub_steps = {"tiny_f32": 200, "decode_top2": 200}
    name = args.workload or workloads.HEADLINE
    res = run_workload(name, args, headline=True)
    variant = (args.backward or args.train or args.router != "topk" or args.router_losses
               or args.k or args.serial or args.drop_policy != "token_order" or args.z_loss
               or args.read_x_rows)
    if args.workload is None and not variant and not args.headline_only:
        # the other four workloads, each measured the same way, as sub-records
        res["workloads"] = {}
        for sub in SUB_WORKLOADS:
            r = run_workload(sub, args, headline=False)
            res["workloads"][sub] = {
                n: r[n] for n in ("value", "unit", "ms_per_step", "steps", "dtype", "config",
                                  "roofline", "layer", "routing", "kernels", "cold_cache",
                                  "cpu_baseline")}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
