"""moe_layer_forward_noalloc (the entry point that allocates nothing) against
moe_layer_forward, through the C ABI.

Both run the same kernels in the same order, so every output must be
identical bit for bit.  Two calls in a row on one device share the library's
scratch array; the second call has a smaller input, so it must not depend on
what the first left behind.  Cases cover a PR-MoE layer with gate priority
and the z-loss (gate-priority segments, z partials in the scratch) and an
int8 layer whose experts run on the per-call XCD schedule (the schedule is
in the scratch too).
"""
import pytest
import torch

from mixture_experts_layer_24_amd import binding, synth, workloads

pytestmark = pytest.mark.gpu

W = workloads.Workload
DEV = "cuda"

FIELDS = ("y", "expert_ids", "gates", "slots", "load", "kept", "aux_loss", "drop_mask",
          "logits", "z_loss")


def _outputs(cfg):
    return binding.alloc_outputs(cfg, DEV, logits=True, x_disp=True, y_disp=True,
                                 dense_out=True, z_loss=True, hidden=True)


def _poison(out):
    for f in ("y", "gates", "logits", "aux_loss", "z_loss", "x_disp", "y_disp", "dense_out"):
        t = getattr(out, f)
        if t is not None:
            t.fill_(float("nan"))
    for f in ("expert_ids", "slots", "load", "kept"):
        getattr(out, f).fill_(-7)
    out.drop_mask.fill_(7)


def _rows_equal(a, b, kept):
    for e, n in enumerate(kept.tolist()):
        if n and not torch.equal(a[e, :n].view(torch.int16), b[e, :n].view(torch.int16)):
            return False
    return True


def _compare(cfg, inp, tag):
    print(f"[no_alloc] {tag}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff} "
          f"wfmt={cfg.expert_wfmt} pr={cfg.pr_moe}", flush=True)
    assert binding.noalloc_scratch_bytes(cfg) <= binding.NOALLOC_SCRATCH_BYTES
    ref = _outputs(cfg)
    ws = binding.alloc_workspace(cfg)
    binding.moe_layer_forward(cfg, inp["x"], inp, ref, ws)
    got = _outputs(cfg)
    _poison(got)
    torch.cuda.synchronize()
    binding.moe_layer_forward_noalloc(cfg, inp["x"], inp, got)
    torch.cuda.synchronize()
    for f in FIELDS:
        a, b = getattr(ref, f), getattr(got, f)
        if a.dtype in (torch.float32, torch.bfloat16):
            a = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16)
            b = b.view(a.dtype)
        assert torch.equal(a, b), f"{tag}: {f} differs from moe_layer_forward"
    assert _rows_equal(ref.x_disp, got.x_disp, ref.kept), f"{tag}: x_disp"
    assert _rows_equal(ref.y_disp, got.y_disp, ref.kept), f"{tag}: y_disp"
    if cfg.pr_moe:
        assert torch.equal(ref.dense_out.view(torch.int16), got.dense_out.view(torch.int16))
    return got


def test_noalloc_matches_layer_forward_prmoe_gate_priority():
    big = W("na_big", T=1000, d=256, E=16, k=2, d_ff=384, capacity_factor=1.0,
            d_ff_dense=256, pr_moe=True, add_skip=True)
    small = W("na_small", T=200, d=128, E=8, k=2, d_ff=192, capacity_factor=0.75,
              d_ff_dense=128, pr_moe=True, add_skip=True)
    for wl, seed in ((big, 1), (small, 2)):
        inp = {k: (None if v is None else v.to(DEV))
               for k, v in synth.make_inputs(wl, seed=seed).items()}
        cfg = binding.config_of(wl, drop_policy="gate_priority")
        got = _compare(cfg, inp, wl.name)
        assert int(got.kept.sum()) < cfg.T * cfg.k  # drops happened


def test_noalloc_matches_layer_forward_int8_schedule():
    big = W("na_i8_big", T=4096, d=256, E=32, k=2, d_ff=256, capacity_factor=1.25,
            wfmt="int8", zipf_s=1.2)
    small = W("na_i8_small", T=2048, d=128, E=32, k=2, d_ff=256, capacity_factor=1.25,
              wfmt="int8", zipf_s=1.2)
    for wl, seed in ((big, 3), (small, 4)):
        inp = {k: (None if v is None else v.to(DEV))
               for k, v in synth.make_inputs(wl, seed=seed).items()}
        cfg = binding.config_of(wl)
        assert binding.capacity(cfg) > 128  # the XCD-scheduled int8 tiles
        _compare(cfg, inp, wl.name)


def test_noalloc_rejects_missing_caller_buffers():
    wl = W("na_args", T=64, d=128, E=4, k=1, d_ff=128, capacity_factor=1.0)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in synth.make_inputs(wl).items()}
    cfg = binding.config_of(wl)
    out = binding.alloc_outputs(cfg, DEV, x_disp=True, y_disp=True)  # no h_disp
    with pytest.raises(binding.MoeError) as ei:
        binding.moe_layer_forward_noalloc(cfg, inp["x"], inp, out)
    assert ei.value.status == binding.MOE_ERR_INVALID_ARG
