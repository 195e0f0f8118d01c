"""CPU oracle for the MoE FFN layer forward -- TEST INFRASTRUCTURE ONLY.

A plain fp64 statement of what the layer computes (``moe_oracle.c``), loaded
through ctypes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
path (the HIP library and its binding) never does.  It shares no code with
the HIP path; the only thing both sides take from a common place is the
seeded input generator, which holds none of the method's arithmetic.

Arrays are numpy arrays (torch CPU tensors are accepted and viewed as numpy):
  float32  -> exact fp32 values
  bfloat16 -> passed as the raw 16-bit patterns (exact)
  int8     -> symmetric int8 codes; their fp16 scales are passed as float32
Every function cites, in ``moe_oracle.c``, the passage of the pages it
follows.

MOE_ORACLE_LIB, when set, names another build of ``moe_oracle.c`` to load;
the mutant test uses it to run the pins against deliberately broken copies.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
and ``tests/test_oracle_bruteforce.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, I8, F64 = 0, 1, 2, 3
DROP_TOKEN_ORDER, DROP_GATE_PRIORITY = 0, 1
ROUTER_TOPK, ROUTER_TOP_P, ROUTER_COSINE, ROUTER_NOISY = 0, 1, 2, 3


def build(out: str = _LIB, src: str = _SRC, extra: tuple = ()) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, IEEE semantics kept)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-Wall", "-Wextra", *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load(path: str | None = None):
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or os.environ.get("MOE_ORACLE_LIB") or _LIB
        if path is None and p == _LIB and (not os.path.exists(p) or
                             os.path.getmtime(p) < os.path.getmtime(_SRC)):
            build(p)
        lib = ctypes.CDLL(p)
        i64, dbl, vp, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.oracle_threads.restype = i32
        lib.oracle_threads.argtypes = []
        lib.oracle_capacity.restype = i64
        lib.oracle_capacity.argtypes = [i64, i64, i64, dbl, i64]
        lib.oracle_route.restype = i32
        lib.oracle_route.argtypes = [i64, i64, i64, i64, i32, vp, i32, vp, i32, vp,
                                     vp, vp, vp, vp]
        lib.oracle_aux_loss.restype = dbl
        lib.oracle_aux_loss.argtypes = [i64, i64, i64, vp, vp, dbl, vp, vp]
        lib.oracle_dispatch.restype = i32
        lib.oracle_dispatch.argtypes = [i64, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp]
        lib.oracle_ffn_rows.restype = i32
        lib.oracle_ffn_rows.argtypes = [i64, i64, i64, vp, i32, vp, vp, i32, vp, vp, vp, vp]
        lib.oracle_combine.restype = i32
        lib.oracle_combine.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_layer_forward.restype = i32
        lib.oracle_layer_forward.argtypes = (
            [i64] * 6 + [dbl, i64] + [i32] * 4 + [dbl, vp, i32, vp, vp, vp, vp, i32, vp, vp,
                                                  vp, vp] + [vp] * 13)
        lib.oracle_layer_backward.restype = i32
        lib.oracle_layer_backward.argtypes = (
            [i64] * 5 + [i64, dbl, i64] + [i32] * 4 + [dbl, vp, i32] + [vp] * 6 +
            [vp, dbl, dbl] + [vp] * 7)
        lib.oracle_backward_sampled.restype = i32
        lib.oracle_backward_sampled.argtypes = (
            [i64] * 6 + [i32] * 3 + [dbl, vp, i32] + [vp] * 6 + [vp, vp, vp, dbl, dbl] +
            [vp, i64, vp, vp, i64, vp, vp, i64, vp])
        lib.oracle_z_loss.restype = dbl
        lib.oracle_z_loss.argtypes = [i64, i64, vp]
        lib.oracle_route_variant.restype = i32
        lib.oracle_route_variant.argtypes = ([i64] * 4 + [i32, i32, dbl, dbl, i64, vp, i32, vp,
                                              vp, vp, vp, vp] + [vp] * 5)
        lib.oracle_importance_load.restype = None
        lib.oracle_importance_load.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_cov2.restype = dbl
        lib.oracle_cov2.argtypes = [i64, vp]
        lib.oracle_layer_forward_v.restype = i32
        lib.oracle_layer_forward_v.argtypes = (
            lib.oracle_layer_forward.argtypes + [i32, dbl, dbl, i64, vp, vp, vp, vp])
        lib.oracle_quantize_sym_int8.restype = i32
        lib.oracle_quantize_sym_int8.argtypes = [i64, i64, vp, vp, vp, vp]
        if path is None:
            _lib = lib
        return lib


# ---------------------------------------------------------------- helpers
def _np(a):
    """numpy view of an array / CPU torch tensor, with its oracle format."""
    try:
        import torch  # noqa: F401
        if isinstance(a, torch.Tensor):
            t = a.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float16:
                return t.float().numpy(), F32
            a = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.int8:
        return a, I8
    if a.dtype == np.float64:
        return a, F64
    raise TypeError(f"unsupported dtype {a.dtype}")


def _scales(s):
    if s is None:
        return None
    s_np, fmt = _np(s)
    if fmt == BF16:
        raise TypeError("scales are fp16 or fp32")
    return np.ascontiguousarray(s_np, dtype=np.float32)


def _p(a):
    return None if a is None else a.ctypes.data


# ---------------------------------------------------------------- stages
def threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().oracle_threads())


def capacity(T: int, E: int, k: int, cf: float, override: int = 0) -> int:
    return int(_load().oracle_capacity(T, E, k, float(cf), int(override)))


def route(x, w_router, k: int, bias=None, normalize: bool = True):
    """logits, probs (T x E fp64), ids (T x k int32), gates (T x k fp64)."""
    xa, xf = _np(x)
    wa, wf = _np(w_router)
    T, d = xa.shape
    E = wa.shape[0]
    assert wa.shape[1] == d
    b = None if bias is None else np.ascontiguousarray(_np(bias)[0], dtype=np.float32)
    logits = np.zeros((T, E)); probs = np.zeros((T, E))
    ids = np.zeros((T, k), np.int32); gates = np.zeros((T, k))
    rc = _load().oracle_route(T, d, E, k, int(normalize), xa.ctypes.data, xf,
                              wa.ctypes.data, wf, _p(b), logits.ctypes.data,
                              probs.ctypes.data, ids.ctypes.data, gates.ctypes.data)
    if rc:
        raise ValueError("oracle_route rejected its arguments")
    return dict(logits=logits, probs=probs, ids=ids, gates=gates)


def aux_loss(ids, probs, alpha: float = 1.0):
    """(loss, f, Q) of the Switch load-balance loss."""
    ids = np.ascontiguousarray(ids, np.int32)
    probs = np.ascontiguousarray(probs, np.float64)
    T, k = ids.shape
    E = probs.shape[1]
    f = np.zeros(E); q = np.zeros(E)
    loss = _load().oracle_aux_loss(T, E, k, ids.ctypes.data, probs.ctypes.data,
                                   float(alpha), f.ctypes.data, q.ctypes.data)
    return loss, f, q


def dispatch(ids, E: int, C: int, gates=None, policy: int = DROP_TOKEN_ORDER):
    """slots (T x k, -1 = dropped), drop (T x k u8), load (E), kept (E)."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    g = None if gates is None else np.ascontiguousarray(gates, np.float64)
    slots = np.zeros((T, k), np.int32); drop = np.zeros((T, k), np.uint8)
    load = np.zeros(E, np.int32); kept = np.zeros(E, np.int32)
    rc = _load().oracle_dispatch(T, E, k, C, ids.ctypes.data, _p(g), policy,
                                 slots.ctypes.data, drop.ctypes.data,
                                 load.ctypes.data, kept.ctypes.data)
    if rc:
        raise ValueError("oracle_dispatch rejected its arguments")
    return dict(slots=slots, drop=drop, load=load, kept=kept)


def ffn_rows(rows, w1, w2, s1=None, s2=None, want_h: bool = False):
    """Two-layer GELU FFN on rows (n x D) with W1 [F, D], W2 [D, F]."""
    ra, rf = _np(rows)
    if ra.ndim == 1:
        ra = ra[None]
    w1a, w1f = _np(w1)
    w2a, w2f = _np(w2)
    assert w1f == w2f
    n, D = ra.shape
    F = w1a.shape[0]
    assert w1a.shape == (F, D) and w2a.shape == (D, F), (w1a.shape, w2a.shape)
    s1a, s2a = _scales(s1), _scales(s2)
    out = np.zeros((n, D))
    h = np.zeros((n, F)) if want_h else None
    rc = _load().oracle_ffn_rows(n, D, F, ra.ctypes.data, rf, w1a.ctypes.data,
                                 w2a.ctypes.data, w1f, _p(s1a), _p(s2a),
                                 out.ctypes.data, _p(h))
    if rc:
        raise ValueError("oracle_ffn_rows rejected its arguments")
    return (out, h) if want_h else out


def combine(slots, gates, expert_out, base=None):
    """y = base + sum over kept assignments of gate * expert output; also M."""
    slots = np.ascontiguousarray(slots, np.int32)
    gates = np.ascontiguousarray(gates, np.float64)
    T, k = slots.shape
    eo = np.ascontiguousarray(expert_out, np.float64)
    D = eo.shape[-1]
    assert eo.shape == (T, k, D)
    b = None if base is None else np.ascontiguousarray(base, np.float64)
    y = np.zeros((T, D)); m = np.zeros((T, D))
    _load().oracle_combine(T, D, k, slots.ctypes.data, gates.ctypes.data,
                           eo.ctypes.data, _p(b), y.ctypes.data, m.ctypes.data)
    return y, m


def z_loss(logits) -> float:
    lg = np.ascontiguousarray(logits, np.float64)
    T, E = lg.shape
    return float(_load().oracle_z_loss(T, E, lg.ctypes.data))


def _router_extras(router, x_fmt, w_noise, noise, emb, T, E, d):
    wn = en = nz = None
    de = 0
    if router == ROUTER_NOISY:
        wn, f = _np(w_noise)
        assert f == x_fmt and wn.shape == (E, d)
        nz = np.ascontiguousarray(_np(noise)[0], dtype=np.float32)
        assert nz.shape == (T, E)
    if router == ROUTER_COSINE:
        en, f = _np(emb)
        assert f == x_fmt and en.shape[0] == E
        de = en.shape[1]
    return wn, nz, en, de


def route_variant(x, w_router, k: int, *, router: int = ROUTER_TOPK, bias=None,
                  normalize: bool = True, top_p: float = 1.0, tau: float = 1.0,
                  w_noise=None, noise=None, emb=None):
    """Router variants (TopK, TopP, cosine with w_router = W_proj [de, d] and
    emb [E, de], noisy TopK with w_noise [E, d] and noise [T, E] fp32):
    logits, probs, ids (-1 = unused slot), gates, load_p (T x E), and the
    per-expert importance and load sums."""
    xa, xf = _np(x)
    wa, wf = _np(w_router)
    assert wf == xf
    T, d = xa.shape
    E = (_np(emb)[0].shape[0] if router == ROUTER_COSINE else wa.shape[0])
    wn, nz, en, de = _router_extras(router, xf, w_noise, noise, emb, T, E, d)
    if router == ROUTER_COSINE:
        assert wa.shape == (de, d)
    b = None if bias is None else np.ascontiguousarray(_np(bias)[0], dtype=np.float32)
    logits = np.zeros((T, E)); probs = np.zeros((T, E)); load_p = np.zeros((T, E))
    ids = np.zeros((T, k), np.int32); gates = np.zeros((T, k))
    rc = _load().oracle_route_variant(T, d, E, k, int(router), int(normalize), float(top_p),
                                      float(tau), de, xa.ctypes.data, xf, wa.ctypes.data, _p(b),
                                      _p(wn), _p(nz), _p(en), logits.ctypes.data,
                                      probs.ctypes.data, ids.ctypes.data, gates.ctypes.data,
                                      load_p.ctypes.data)
    if rc:
        raise ValueError("oracle_route_variant rejected its arguments")
    imp, load = importance_load(ids, gates, load_p)
    return dict(logits=logits, probs=probs, ids=ids, gates=gates, load_p=load_p,
                importance=imp, load=load)


def importance_load(ids, gates, load_p):
    """Per-expert Importance (sum of gates) and Load (sum of P(x, e))."""
    ids = np.ascontiguousarray(ids, np.int32)
    gates = np.ascontiguousarray(gates, np.float64)
    load_p = np.ascontiguousarray(load_p, np.float64)
    T, k = ids.shape
    E = load_p.shape[1]
    imp = np.zeros(E); load = np.zeros(E)
    _load().oracle_importance_load(T, E, k, ids.ctypes.data, gates.ctypes.data,
                                   load_p.ctypes.data, imp.ctypes.data, load.ctypes.data)
    return imp, load


def cov2(v) -> float:
    """Squared coefficient of variation (population variance / mean^2)."""
    v = np.ascontiguousarray(v, np.float64)
    return float(_load().oracle_cov2(v.size, v.ctypes.data))


def quantize_sym_int8(w, scale=None):
    """(codes int8 [N, K], scales fp64 [N, K/128]) of an fp64 matrix."""
    w = np.ascontiguousarray(w, np.float64)
    N, K = w.shape
    q = np.zeros((N, K), np.int8)
    s_out = np.zeros((N, K // 128))
    s_in = None if scale is None else np.ascontiguousarray(scale, np.float64)
    rc = _load().oracle_quantize_sym_int8(N, K, w.ctypes.data, _p(s_in),
                                          q.ctypes.data, s_out.ctypes.data)
    if rc:
        raise ValueError("K must be a multiple of 128")
    return q, s_out


def layer_forward(x, w_router, w1, w2, *, k: int, capacity_factor: float,
                  capacity_override: int = 0, bias=None, s1=None, s2=None,
                  wm1=None, wm2=None, normalize: bool = True, pr_moe: bool = False,
                  add_skip: bool = True, policy: int = DROP_TOKEN_ORDER,
                  alpha: float = 1.0, router: int = ROUTER_TOPK, top_p: float = 1.0,
                  tau: float = 1.0, w_noise=None, noise=None, emb=None):
    """Whole layer; returns a dict of every intermediate the layer defines.
    router / top_p / tau / w_noise / noise / emb: as route_variant (for the
    cosine router w_router is W_proj)."""
    xa, xf = _np(x)
    wra, wrf = _np(w_router)
    assert wrf == xf, "router weights share the activation format"
    w1a, wf = _np(w1)
    w2a, wf2 = _np(w2)
    assert wf == wf2
    T, D = xa.shape
    E, F = w1a.shape[0], w1a.shape[1]
    assert w1a.shape == (E, F, D) and w2a.shape == (E, D, F)
    wn, nz, en, de = _router_extras(router, xf, w_noise, noise, emb, T, E, D)
    Fd = 0
    wm1a = wm2a = None
    if pr_moe:
        wm1a, f1 = _np(wm1)
        wm2a, f2 = _np(wm2)
        assert f1 == xf and f2 == xf
        Fd = wm1a.shape[0]
        assert wm1a.shape == (Fd, D) and wm2a.shape == (D, Fd)
    b = None if bias is None else np.ascontiguousarray(_np(bias)[0], dtype=np.float32)
    s1a, s2a = _scales(s1), _scales(s2)
    out = dict(
        logits=np.zeros((T, E)), probs=np.zeros((T, E)),
        ids=np.zeros((T, k), np.int32), gates=np.zeros((T, k)),
        slots=np.zeros((T, k), np.int32), drop=np.zeros((T, k), np.uint8),
        load=np.zeros(E, np.int32), kept=np.zeros(E, np.int32),
        expert_out=np.zeros((T, k, D)), m=np.zeros((T, D)), dense=np.zeros((T, D)),
        y=np.zeros((T, D)), aux=np.zeros(1), load_p=np.zeros((T, E)))
    rc = _load().oracle_layer_forward_v(
        T, D, E, k, F, Fd, float(capacity_factor), int(capacity_override),
        int(normalize), int(pr_moe), int(add_skip), int(policy), float(alpha),
        xa.ctypes.data, xf, wra.ctypes.data, _p(b), w1a.ctypes.data,
        w2a.ctypes.data, wf, _p(s1a), _p(s2a), _p(wm1a), _p(wm2a),
        *(out[n].ctypes.data for n in ("logits", "probs", "ids", "gates", "slots",
                                       "drop", "load", "kept", "expert_out", "m",
                                       "dense", "y", "aux")),
        int(router), float(top_p), float(tau), de, _p(wn), _p(nz), _p(en),
        out["load_p"].ctypes.data)
    if rc:
        raise ValueError("oracle_layer_forward rejected its arguments")
    out["aux"] = float(out["aux"][0])
    out["capacity"] = capacity(T, E, k, capacity_factor, capacity_override)
    return out


def layer_backward(x, w_router, w1, w2, dy, *, k: int, capacity_factor: float,
                   capacity_override: int = 0, bias=None, wm1=None, wm2=None,
                   normalize: bool = True, pr_moe: bool = False, add_skip: bool = True,
                   policy: int = DROP_TOKEN_ORDER, alpha: float = 1.0, g_aux: float = 0.0,
                   g_z: float = 0.0):
    """Gradients of <dy, y> + g_aux * aux + g_z * z_loss with respect to x and
    every weight (plain weights in the activation format); returns a dict."""
    xa, xf = _np(x)
    wra, wrf = _np(w_router)
    w1a, f1 = _np(w1)
    w2a, f2 = _np(w2)
    assert wrf == xf and f1 == xf and f2 == xf, "the backward takes one format"
    T, D = xa.shape
    E, F = w1a.shape[0], w1a.shape[1]
    Fd = 0
    m1 = m2 = None
    if pr_moe:
        m1, fm1 = _np(wm1)
        m2, fm2 = _np(wm2)
        assert fm1 == xf and fm2 == xf
        Fd = m1.shape[0]
    b = None if bias is None else np.ascontiguousarray(_np(bias)[0], dtype=np.float32)
    g = np.ascontiguousarray(np.asarray(dy, dtype=np.float64).reshape(T, D))
    out = dict(dx=np.zeros((T, D)), dw_router=np.zeros((E, D)), db_router=np.zeros(E),
               dw1=np.zeros((E, F, D)), dw2=np.zeros((E, D, F)),
               dwm1=np.zeros((max(Fd, 1), D)), dwm2=np.zeros((D, max(Fd, 1))))
    rc = _load().oracle_layer_backward(
        T, D, E, k, F, Fd, float(capacity_factor), int(capacity_override), int(normalize),
        int(pr_moe), int(add_skip), int(policy), float(alpha), xa.ctypes.data, xf,
        wra.ctypes.data, _p(b), w1a.ctypes.data, w2a.ctypes.data, _p(m1), _p(m2),
        g.ctypes.data, float(g_aux), float(g_z), out["dx"].ctypes.data,
        out["dw_router"].ctypes.data, out["db_router"].ctypes.data, out["dw1"].ctypes.data,
        out["dw2"].ctypes.data, out["dwm1"].ctypes.data, out["dwm2"].ctypes.data)
    if rc:
        raise ValueError("oracle_layer_backward rejected its arguments")
    if not pr_moe:
        out["dwm1"] = out["dwm2"] = None
    return out


def backward_sampled(x, w_router, w1, w2, ids, slots, dy, rows, *, k: int, bias=None,
                     wm1=None, wm2=None, normalize: bool = True, pr_moe: bool = False,
                     add_skip: bool = True, alpha: float = 1.0, g_aux: float = 0.0,
                     g_z: float = 0.0, dw1_idx=(), dw2_idx=()):
    """dx rows of the tokens `rows` and dW1 / dW2 entries (triples (e, f, i) /
    (e, o, f)) of the layer backward under the given routing decisions
    ids / slots (T x k); dy: T x D upstream gradient."""
    xa, xf = _np(x)
    wra, _ = _np(w_router)
    w1a, _ = _np(w1)
    w2a, _ = _np(w2)
    T, D = xa.shape
    E, F = w1a.shape[0], w1a.shape[1]
    Fd = 0
    m1 = m2 = None
    if pr_moe:
        m1, _ = _np(wm1)
        m2, _ = _np(wm2)
        Fd = m1.shape[0]
    b = None if bias is None else np.ascontiguousarray(_np(bias)[0], dtype=np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    slots = np.ascontiguousarray(slots, np.int32)
    rows = np.ascontiguousarray(rows, np.int64)
    dyf = np.ascontiguousarray(np.asarray(dy, np.float64).reshape(T, D))
    i1 = np.ascontiguousarray(np.asarray(dw1_idx, np.int64).reshape(-1, 3))
    i2 = np.ascontiguousarray(np.asarray(dw2_idx, np.int64).reshape(-1, 3))
    dx = np.zeros((len(rows), D))
    v1, v2 = np.zeros(len(i1)), np.zeros(len(i2))
    rc = _load().oracle_backward_sampled(
        T, D, E, k, F, Fd, int(normalize), int(pr_moe), int(add_skip), float(alpha),
        xa.ctypes.data, xf, wra.ctypes.data, _p(b), w1a.ctypes.data, w2a.ctypes.data,
        _p(m1), _p(m2), ids.ctypes.data, slots.ctypes.data, dyf.ctypes.data, float(g_aux),
        float(g_z), rows.ctypes.data, len(rows), dx.ctypes.data, i1.ctypes.data, len(i1),
        v1.ctypes.data, i2.ctypes.data, len(i2), v2.ctypes.data)
    if rc:
        raise ValueError("oracle_backward_sampled rejected its arguments")
    return dict(dx=dx, dw1=v1, dw2=v2)
