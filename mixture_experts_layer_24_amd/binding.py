"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every step of the layer runs in the HIP library ``libmoe_mi355x.so``; this
module checks dtypes, shapes and devices of torch tensors, passes their
device pointers and torch's current HIP stream, and turns a non-zero status
into ``MoeError``.  torch provides device memory and streams, nothing else.
If the library is missing, ``lib()`` raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading

import torch

from .workloads import Workload

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES
MOE_F32, MOE_BF16 = 0, 1
MOE_W_PLAIN, MOE_W_INT8_G128, MOE_W_BF16_PACKED = 0, 1, 2
WFMTS = {"plain": MOE_W_PLAIN, "int8": MOE_W_INT8_G128, "packed": MOE_W_BF16_PACKED}
MOE_DROP_TOKEN_ORDER = 0
MOE_DROP_GATE_PRIORITY = 1
ENTRY_ROUTE, ENTRY_DISPATCH, ENTRY_EXPERT_FFN, ENTRY_COMBINE, ENTRY_LAYER, ENTRY_BACKWARD = \
    range(6)

EXPORTED = ("moe_capacity", "moe_workspace_bytes", "moe_route", "moe_route_ex", "moe_dispatch",
            "moe_expert_ffn", "moe_dense_mlp", "moe_combine", "moe_layer_forward",
            "moe_layer_backward", "moe_pack_expert_weights", "moe_layer_forward_noalloc",
            "moe_layer_forward_noalloc_scratch_bytes",
            "moe_status_string", "moe_profile_enable", "moe_profile_filter", "moe_profile_reset",
            "moe_profile_read")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} ({status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("d_ff", ctypes.c_int64), ("d_ff_dense", ctypes.c_int64),
                ("capacity_factor", ctypes.c_double), ("capacity", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("expert_wfmt", ctypes.c_int32),
                ("normalize_topk", ctypes.c_int32), ("pr_moe", ctypes.c_int32),
                ("add_skip", ctypes.c_int32), ("drop_policy", ctypes.c_int32),
                ("aux_alpha", ctypes.c_float), ("overlap_dense", ctypes.c_int32),
                ("router", ctypes.c_int32), ("top_p", ctypes.c_float), ("cos_tau", ctypes.c_float),
                ("cos_dim", ctypes.c_int32), ("w_importance", ctypes.c_float),
                ("w_load", ctypes.c_float), ("read_x_rows", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w1", "w1_scale", "w2", "w2_scale", "wm1", "wm2",
                 "w_noise", "w_proj", "expert_emb", "noise")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "db_router", "dw1", "dw2", "dwm1", "dwm2")]


class Outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("y", "expert_ids", "gates", "slots", "load", "kept", "aux_loss", "drop_mask",
                 "logits", "x_disp", "y_disp", "dense_out", "z_loss", "h_disp", "z_disp",
                 "h_dense", "z_dense", "importance_loss", "load_loss")]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m mixture_experts_layer_24_amd.build` (no fallback exists)")
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
            cfgp = ctypes.POINTER(Config)
            L.moe_capacity.restype = i64
            L.moe_capacity.argtypes = [cfgp]
            L.moe_workspace_bytes.restype = sz
            L.moe_workspace_bytes.argtypes = [cfgp, i32]
            L.moe_route.restype = i32
            L.moe_route.argtypes = [cfgp] + [vp] * 8 + [vp, sz, vp]
            L.moe_dispatch.restype = i32
            L.moe_dispatch.argtypes = [cfgp] + [vp] * 8 + [vp, sz, vp]
            L.moe_expert_ffn.restype = i32
            L.moe_expert_ffn.argtypes = [cfgp] + [vp] * 7 + [vp, sz, vp]
            L.moe_dense_mlp.restype = i32
            L.moe_dense_mlp.argtypes = [cfgp] + [vp] * 4 + [vp, sz, vp]
            L.moe_combine.restype = i32
            L.moe_combine.argtypes = [cfgp] + [vp] * 7 + [vp]
            L.moe_layer_forward.restype = i32
            L.moe_layer_forward.argtypes = [cfgp, vp, ctypes.POINTER(Weights),
                                            ctypes.POINTER(Outputs), vp, sz, vp]
            L.moe_layer_forward_noalloc.restype = i32
            L.moe_layer_forward_noalloc.argtypes = [cfgp, vp, ctypes.POINTER(Weights),
                                                    ctypes.POINTER(Outputs), vp]
            L.moe_layer_forward_noalloc_scratch_bytes.restype = sz
            L.moe_layer_forward_noalloc_scratch_bytes.argtypes = [cfgp]
            L.moe_route_ex.restype = i32
            L.moe_route_ex.argtypes = [cfgp, vp, ctypes.POINTER(Weights),
                                       ctypes.POINTER(Outputs), vp, sz, vp]
            L.moe_layer_backward.restype = i32
            L.moe_layer_backward.argtypes = [cfgp, vp, ctypes.POINTER(Weights),
                                             ctypes.POINTER(Outputs), vp, ctypes.c_float,
                                             ctypes.c_float, ctypes.POINTER(Grads), vp, sz, vp]
            L.moe_status_string.restype = ctypes.c_char_p
            L.moe_status_string.argtypes = [i32]
            L.moe_profile_enable.restype = i32
            L.moe_profile_enable.argtypes = [i32]
            L.moe_pack_expert_weights.restype = i32
            L.moe_pack_expert_weights.argtypes = [cfgp, i32, vp, vp, vp]
            L.moe_profile_filter.restype = i32
            L.moe_profile_filter.argtypes = [ctypes.c_char_p]
            L.moe_profile_reset.restype = i32
            L.moe_profile_reset.argtypes = []
            L.moe_profile_read.restype = i32
            L.moe_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_double), i32]
            _lib = L
        return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, status_string(status))


# ------------------------------------------------------------------ config
ROUTERS = {"topk": 0, "top_p": 1, "cosine": 2, "noisy_topk": 3}


def make_config(*, T, d, E, k, d_ff, capacity_factor=1.0, capacity=0, act="bf16",
                wfmt="plain", d_ff_dense=0, pr_moe=False, add_skip=True,
                normalize_topk=True, aux_alpha=1.0, overlap_dense=True,
                drop_policy="token_order", router="topk", top_p=0.0, cos_tau=0.0,
                cos_dim=0, w_importance=0.0, w_load=0.0, read_x_rows=False) -> Config:
    if drop_policy not in ("token_order", "gate_priority"):
        raise ValueError(f"drop_policy {drop_policy!r}")
    if router not in ROUTERS:
        raise ValueError(f"router {router!r}")
    if wfmt not in WFMTS:
        raise ValueError(f"wfmt {wfmt!r}")
    return Config(T=T, d=d, E=E, k=k, d_ff=d_ff, d_ff_dense=d_ff_dense,
                  capacity_factor=capacity_factor, capacity=capacity,
                  act_dtype=MOE_F32 if act == "f32" else MOE_BF16,
                  expert_wfmt=WFMTS[wfmt],
                  normalize_topk=int(normalize_topk), pr_moe=int(pr_moe),
                  add_skip=int(add_skip),
                  drop_policy=(MOE_DROP_GATE_PRIORITY if drop_policy == "gate_priority"
                               else MOE_DROP_TOKEN_ORDER),
                  aux_alpha=aux_alpha, overlap_dense=int(overlap_dense),
                  router=ROUTERS[router], top_p=top_p, cos_tau=cos_tau, cos_dim=cos_dim,
                  w_importance=w_importance, w_load=w_load, read_x_rows=int(read_x_rows))


def config_of(wl: Workload, **override) -> Config:
    kw = dict(T=wl.T, d=wl.d, E=wl.E, k=wl.k, d_ff=wl.d_ff,
              capacity_factor=wl.capacity_factor, act=wl.act, wfmt=wl.wfmt,
              d_ff_dense=wl.d_ff_dense, pr_moe=wl.pr_moe, add_skip=wl.add_skip,
              normalize_topk=wl.normalize_topk, aux_alpha=wl.aux_alpha)
    kw.update(override)
    return make_config(**kw)


def capacity(cfg: Config) -> int:
    c = lib().moe_capacity(ctypes.byref(cfg))
    if c < 0:
        _check("moe_capacity", int(c))
    return int(c)


def workspace_bytes(cfg: Config, entry: int = ENTRY_LAYER) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), entry))


# ------------------------------------------------------------------ marshalling
def _act_dtype(cfg: Config):
    return torch.float32 if cfg.act_dtype == MOE_F32 else torch.bfloat16


def _ptr(t, shape=None, dtype=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, dtype=torch.uint8, name="ws"), ws.numel()


def alloc_workspace(cfg: Config, entry: int = ENTRY_LAYER, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(cfg, entry), 1), dtype=torch.uint8, device=device)


def _wdtype(cfg):
    return torch.int8 if cfg.expert_wfmt == MOE_W_INT8_G128 else _act_dtype(cfg)


# ------------------------------------------------------------------ entry points
def moe_route(cfg, x, w_router, b_router, expert_ids, gates, logits, aux_loss, ws,
              stream=None, z_loss=None):
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    a = _act_dtype(cfg)
    wsp, wsn = _ws(ws)
    _check("moe_route", lib().moe_route(
        ctypes.byref(cfg), _ptr(x, (T, d), a, "x"), _ptr(w_router, (E, d), a, "w_router"),
        _ptr(b_router, (E,), torch.float32, "b_router", True),
        _ptr(expert_ids, (T, k), torch.int32, "expert_ids"),
        _ptr(gates, (T, k), torch.float32, "gates"),
        _ptr(logits, (T, E), torch.float32, "logits", True),
        _ptr(aux_loss, (1,), torch.float32, "aux_loss"),
        _ptr(z_loss, (1,), torch.float32, "z_loss", True), wsp, wsn, _stream(stream)))


def moe_dispatch(cfg, x, expert_ids, slots, drop_mask, load, kept, x_disp, ws, stream=None,
                 gates=None):
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    C = capacity(cfg)
    a = _act_dtype(cfg)
    wsp, wsn = _ws(ws)
    gp = cfg.drop_policy == MOE_DROP_GATE_PRIORITY
    _check("moe_dispatch", lib().moe_dispatch(
        ctypes.byref(cfg), _ptr(x, (T, d), a, "x"),
        _ptr(expert_ids, (T, k), torch.int32, "expert_ids"),
        _ptr(gates, (T, k), torch.float32, "gates", not gp),
        _ptr(slots, (T, k), torch.int32, "slots"),
        _ptr(drop_mask, (T, k), torch.uint8, "drop_mask", True),
        _ptr(load, (E,), torch.int32, "load"), _ptr(kept, (E,), torch.int32, "kept"),
        _ptr(x_disp, (E, C, d), a, "x_disp"), wsp, wsn, _stream(stream)))


def moe_expert_ffn(cfg, x_disp, kept, w1, w1_scale, w2, w2_scale, y_disp, ws, stream=None):
    d, E, F = cfg.d, cfg.E, cfg.d_ff
    C = capacity(cfg)
    a, wd = _act_dtype(cfg), _wdtype(cfg)
    q8 = cfg.expert_wfmt == MOE_W_INT8_G128
    wsp, wsn = _ws(ws)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(cfg), _ptr(x_disp, (E, C, d), a, "x_disp"),
        _ptr(kept, (E,), torch.int32, "kept"), _ptr(w1, (E, F, d), wd, "w1"),
        _ptr(w1_scale, (E, F, d // 128), torch.float16, "w1_scale", not q8),
        _ptr(w2, (E, d, F), wd, "w2"),
        _ptr(w2_scale, (E, d, F // 128), torch.float16, "w2_scale", not q8),
        _ptr(y_disp, (E, C, d), a, "y_disp"), wsp, wsn, _stream(stream)))


def pack_expert_weights(cfg, which, w, out=None, stream=None):
    """Row-major bf16 expert weights (which = 1: W1 [E, d_ff, d]; 2: W2 [E, d,
    d_ff]) in MOE_W_BF16_PACKED order, in a tensor of the same shape."""
    shape = (cfg.E, cfg.d_ff, cfg.d) if which == 1 else (cfg.E, cfg.d, cfg.d_ff)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    _check("moe_pack_expert_weights", lib().moe_pack_expert_weights(
        ctypes.byref(cfg), which, _ptr(w, shape, torch.bfloat16, "w"),
        _ptr(out, shape, torch.bfloat16, "w_packed"), _stream(stream)))
    return out


def moe_dense_mlp(cfg, x, wm1, wm2, dense_out, ws, stream=None):
    T, d, Fd = cfg.T, cfg.d, cfg.d_ff_dense
    a = _act_dtype(cfg)
    wsp, wsn = _ws(ws)
    _check("moe_dense_mlp", lib().moe_dense_mlp(
        ctypes.byref(cfg), _ptr(x, (T, d), a, "x"), _ptr(wm1, (Fd, d), a, "wm1"),
        _ptr(wm2, (d, Fd), a, "wm2"), _ptr(dense_out, (T, d), a, "dense_out"), wsp, wsn,
        _stream(stream)))


def moe_combine(cfg, y_disp, expert_ids, slots, gates, base, base2, y, stream=None):
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    C = capacity(cfg)
    a = _act_dtype(cfg)
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(cfg), _ptr(y_disp, (E, C, d), a, "y_disp"),
        _ptr(expert_ids, (T, k), torch.int32, "expert_ids"),
        _ptr(slots, (T, k), torch.int32, "slots"), _ptr(gates, (T, k), torch.float32, "gates"),
        _ptr(base, (T, d), a, "base", True), _ptr(base2, (T, d), a, "base2", True),
        _ptr(y, (T, d), a, "y"), _stream(stream)))


@dataclasses.dataclass
class LayerOutputs:
    y: torch.Tensor
    expert_ids: torch.Tensor
    gates: torch.Tensor
    slots: torch.Tensor
    load: torch.Tensor
    kept: torch.Tensor
    aux_loss: torch.Tensor
    drop_mask: torch.Tensor | None = None
    logits: torch.Tensor | None = None
    x_disp: torch.Tensor | None = None
    y_disp: torch.Tensor | None = None
    dense_out: torch.Tensor | None = None
    z_loss: torch.Tensor | None = None
    h_disp: torch.Tensor | None = None   # [E, C, d_ff] GELU(W1 x), kept rows
    z_disp: torch.Tensor | None = None   # [E, C, d_ff] W1 x
    h_dense: torch.Tensor | None = None  # [T, d_ff_dense] (pr_moe)
    z_dense: torch.Tensor | None = None
    importance_loss: torch.Tensor | None = None
    load_loss: torch.Tensor | None = None


def alloc_outputs(cfg: Config, device="cuda", *, drop_mask=True, logits=False,
                  x_disp=False, y_disp=False, dense_out=False, z_loss=False,
                  saved_activations=False, importance_loss=False,
                  load_loss=False, hidden=False) -> LayerOutputs:
    """saved_activations: also keep the FFN hidden activations and their
    pre-activations, which the backward then reads instead of recomputing.
    hidden: caller-owned hidden rows (h_disp, and h_dense for PR-MoE) without
    the pre-activations."""
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    C = capacity(cfg)
    a = _act_dtype(cfg)
    e = lambda *s, dt=a: torch.empty(s, dtype=dt, device=device)  # noqa: E731
    return LayerOutputs(
        y=e(T, d), expert_ids=e(T, k, dt=torch.int32), gates=e(T, k, dt=torch.float32),
        slots=e(T, k, dt=torch.int32), load=e(E, dt=torch.int32), kept=e(E, dt=torch.int32),
        aux_loss=e(1, dt=torch.float32),
        drop_mask=e(T, k, dt=torch.uint8) if drop_mask else None,
        logits=e(T, E, dt=torch.float32) if logits else None,
        x_disp=e(E, C, d) if x_disp else None, y_disp=e(E, C, d) if y_disp else None,
        dense_out=e(T, d) if (dense_out and cfg.pr_moe) else None,
        z_loss=e(1, dt=torch.float32) if z_loss else None,
        h_disp=e(E, C, cfg.d_ff) if (saved_activations or hidden) else None,
        z_disp=e(E, C, cfg.d_ff) if saved_activations else None,
        h_dense=(e(T, cfg.d_ff_dense) if ((saved_activations or hidden) and cfg.pr_moe)
                 else None),
        z_dense=e(T, cfg.d_ff_dense) if (saved_activations and cfg.pr_moe) else None,
        importance_loss=e(1, dt=torch.float32) if importance_loss else None,
        load_loss=e(1, dt=torch.float32) if load_loss else None)


def moe_layer_forward(cfg, x, weights: dict, out: LayerOutputs, ws, stream=None):
    """weights: dict with w_router, b_router, w1, w1_scale, w2, w2_scale, wm1, wm2."""
    W, O = _weights_struct(cfg, weights), _outputs_struct(cfg, out)
    wsp, wsn = _ws(ws)
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(cfg), _ptr(x, (cfg.T, cfg.d), _act_dtype(cfg), "x"), ctypes.byref(W),
        ctypes.byref(O), wsp, wsn, _stream(stream)))


def noalloc_scratch_bytes(cfg: Config) -> int:
    """Scratch bytes moe_layer_forward_noalloc needs for cfg."""
    return int(lib().moe_layer_forward_noalloc_scratch_bytes(ctypes.byref(cfg)))


def moe_layer_forward_noalloc(cfg, x, weights: dict, out: LayerOutputs, stream=None):
    """The layer without a workspace: out must hold x_disp, y_disp and h_disp
    (and dense_out and h_dense for PR-MoE); the library's own per-device
    scratch holds the rest."""
    W, O = _weights_struct(cfg, weights), _outputs_struct(cfg, out)
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(cfg), _ptr(x, (cfg.T, cfg.d), _act_dtype(cfg), "x"), ctypes.byref(W),
        ctypes.byref(O), _stream(stream)))


def moe_route_ex(cfg, x, weights: dict, out: LayerOutputs, ws, stream=None):
    """Any router (cfg.router): writes out.expert_ids, gates, aux_loss and the
    optional logits, z_loss, importance_loss and load_loss."""
    W, O = _weights_struct(cfg, weights, router_only=True), _outputs_struct(cfg, out,
                                                                             router_only=True)
    wsp, wsn = _ws(ws)
    _check("moe_route_ex", lib().moe_route_ex(
        ctypes.byref(cfg), _ptr(x, (cfg.T, cfg.d), _act_dtype(cfg), "x"), ctypes.byref(W),
        ctypes.byref(O), wsp, wsn, _stream(stream)))


@dataclasses.dataclass
class LayerGrads:
    dx: torch.Tensor
    dw_router: torch.Tensor
    dw1: torch.Tensor
    dw2: torch.Tensor
    db_router: torch.Tensor | None = None
    dwm1: torch.Tensor | None = None
    dwm2: torch.Tensor | None = None


def alloc_grads(cfg: Config, device="cuda", *, db_router=True) -> LayerGrads:
    T, d, E, F, Fd = cfg.T, cfg.d, cfg.E, cfg.d_ff, cfg.d_ff_dense
    a = _act_dtype(cfg)
    e = lambda *s, dt=a: torch.empty(s, dtype=dt, device=device)  # noqa: E731
    pr = bool(cfg.pr_moe)
    return LayerGrads(dx=e(T, d), dw_router=e(E, d), dw1=e(E, F, d), dw2=e(E, d, F),
                      db_router=e(E, dt=torch.float32) if db_router else None,
                      dwm1=e(Fd, d) if pr else None, dwm2=e(d, Fd) if pr else None)


def moe_layer_backward(cfg, x, weights: dict, fwd: LayerOutputs, dy, grads: LayerGrads, ws,
                       g_aux: float = 0.0, g_z: float = 0.0, stream=None):
    """Backward of moe_layer_forward (fwd: its outputs, with logits, x_disp and
    y_disp allocated)."""
    T, d, E, F, Fd = cfg.T, cfg.d, cfg.E, cfg.d_ff, cfg.d_ff_dense
    a = _act_dtype(cfg)
    pr = bool(cfg.pr_moe)
    W, O = _weights_struct(cfg, weights), _outputs_struct(cfg, fwd)
    G = Grads(dx=_ptr(grads.dx, (T, d), a, "dx"),
              dw_router=_ptr(grads.dw_router, (E, d), a, "dw_router"),
              db_router=_ptr(grads.db_router, (E,), torch.float32, "db_router", True),
              dw1=_ptr(grads.dw1, (E, F, d), a, "dw1"), dw2=_ptr(grads.dw2, (E, d, F), a, "dw2"),
              dwm1=_ptr(grads.dwm1, (Fd, d), a, "dwm1", not pr),
              dwm2=_ptr(grads.dwm2, (d, Fd), a, "dwm2", not pr))
    wsp, wsn = _ws(ws)
    _check("moe_layer_backward", lib().moe_layer_backward(
        ctypes.byref(cfg), _ptr(x, (T, d), a, "x"), ctypes.byref(W), ctypes.byref(O),
        _ptr(dy, (T, d), a, "dy"), float(g_aux), float(g_z), ctypes.byref(G), wsp, wsn,
        _stream(stream)))


def _weights_struct(cfg, weights: dict, router_only: bool = False) -> Weights:
    T, d, E, k, F, Fd = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.d_ff_dense
    C = capacity(cfg)
    a, wd = _act_dtype(cfg), _wdtype(cfg)
    q8 = cfg.expert_wfmt == MOE_W_INT8_G128
    pr = bool(cfg.pr_moe)
    cos, noisy = cfg.router == ROUTERS["cosine"], cfg.router == ROUTERS["noisy_topk"]
    W = Weights(
        w_router=_ptr(weights.get("w_router"), (E, d), a, "w_router", cos),
        b_router=_ptr(weights.get("b_router"), (E,), torch.float32, "b_router", True),
        w1=_ptr(weights.get("w1"), (E, F, d), wd, "w1", router_only),
        w1_scale=_ptr(weights.get("w1_scale"), (E, F, d // 128), torch.float16, "w1_scale",
                      not q8),
        w2=_ptr(weights.get("w2"), (E, d, F), wd, "w2", router_only),
        w2_scale=_ptr(weights.get("w2_scale"), (E, d, F // 128), torch.float16, "w2_scale",
                      not q8),
        wm1=_ptr(weights.get("wm1"), (Fd, d), a, "wm1", not pr),
        wm2=_ptr(weights.get("wm2"), (d, Fd), a, "wm2", not pr),
        w_noise=_ptr(weights.get("w_noise"), (E, d), a, "w_noise", not noisy),
        noise=_ptr(weights.get("noise"), (T, E), torch.float32, "noise", not noisy),
        w_proj=_ptr(weights.get("w_proj"), (cfg.cos_dim, d), a, "w_proj", not cos),
        expert_emb=_ptr(weights.get("expert_emb"), (E, cfg.cos_dim), a, "expert_emb", not cos))
    return W


def _outputs_struct(cfg, out: LayerOutputs, router_only: bool = False) -> Outputs:
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    C = capacity(cfg)
    a = _act_dtype(cfg)
    return Outputs(
        y=_ptr(out.y, (T, d), a, "y", router_only),
        expert_ids=_ptr(out.expert_ids, (T, k), torch.int32, "expert_ids"),
        gates=_ptr(out.gates, (T, k), torch.float32, "gates"),
        slots=_ptr(out.slots, (T, k), torch.int32, "slots", router_only),
        load=_ptr(out.load, (E,), torch.int32, "load", router_only),
        kept=_ptr(out.kept, (E,), torch.int32, "kept", router_only),
        aux_loss=_ptr(out.aux_loss, (1,), torch.float32, "aux_loss"),
        drop_mask=_ptr(out.drop_mask, (T, k), torch.uint8, "drop_mask", True),
        logits=_ptr(out.logits, (T, E), torch.float32, "logits", True),
        x_disp=_ptr(out.x_disp, (E, C, d), a, "x_disp", True),
        y_disp=_ptr(out.y_disp, (E, C, d), a, "y_disp", True),
        dense_out=_ptr(out.dense_out, (T, d), a, "dense_out", True),
        z_loss=_ptr(out.z_loss, (1,), torch.float32, "z_loss", True),
        h_disp=_ptr(out.h_disp, (E, C, cfg.d_ff), a, "h_disp", True),
        z_disp=_ptr(out.z_disp, (E, C, cfg.d_ff), a, "z_disp", True),
        h_dense=_ptr(out.h_dense, (T, cfg.d_ff_dense), a, "h_dense", True),
        z_dense=_ptr(out.z_dense, (T, cfg.d_ff_dense), a, "z_dense", True),
        importance_loss=_ptr(out.importance_loss, (1,), torch.float32, "importance_loss", True),
        load_loss=_ptr(out.load_loss, (1,), torch.float32, "load_loss", True))


# ------------------------------------------------------------------ profiling
def profile_enable(on: bool = True):
    lib().moe_profile_enable(int(on))


def profile_filter(name=None):
    """Time only launches named `name` ("role:tile"); None times every launch."""
    lib().moe_profile_filter(None if not name else name.encode())


def profile_reset():
    lib().moe_profile_reset()


def profile_read(cap: int = 64) -> dict:
    """{kernel name: (launches, total ms)} since the last read/reset."""
    names = ctypes.create_string_buffer(64 * cap)
    n_l = (ctypes.c_int64 * cap)()
    ms = (ctypes.c_double * cap)()
    n = lib().moe_profile_read(names, n_l, ms, cap)
    out = {}
    for i in range(min(n, cap)):
        nm = names.raw[64 * i: 64 * i + 64].split(b"\0", 1)[0].decode()
        out[nm] = (int(n_l[i]), float(ms[i]))
    return out
