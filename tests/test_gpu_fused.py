"""The forward as one kernel launch (moe_layer_forward) against the per-step calls
(moe_route, moe_dispatch, moe_expert_ffn, moe_combine) and against the oracle.

Every step of the single launch runs the same device code as its own kernel, so every output
-- routing, permutation, dispatched rows, the saved g|u and h, the expert outputs and the
layer output -- must be bit-identical to the per-step forward's, at reduced sizes and at the
full workload sizes.  The reduced cases are also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_39_amd as moe
import oracle as orc
import workloads as wk
from gpu_harness import TOL_BF16, assert_close, bf, digest, host, oracle_params
from mixture_experts_layer_39_amd.layer import LayerCfg, MoELayer

pytestmark = pytest.mark.gpu

REDUCED = {  # case: (workload, reduced sizes)
    "tiny_t128": ("tiny_t128", dict()),
    "tiny_t1": ("tiny_t128", dict(T=1)),
    "tiny_t3_k1": ("tiny_t128", dict(T=3, k=1)),
    "mid_t2048": ("mid_t2048", dict(T=384, H=1024, E=8, I=384, Is=256)),
    "dsv3_ep64": ("dsv3_ep64", dict(T=256, H=1024, I=512, R_share=2048)),
    "dsv3_e256_zipf": ("dsv3_e256_zipf", dict(T=512, H=512, E=64, I=256, Is=256, minibatch=0)),
}
FULL = {
    "mid_t2048": ("mid_t2048", dict()),
    "dsv3_ep64": ("dsv3_ep64", dict()),
    "dsv3_e256_zipf_unstreamed": ("dsv3_e256_zipf", dict(T=2048, minibatch=0)),
}


def _wl(case):
    base, kw = case
    return wk.WORKLOADS[base].scaled(**kw)


def _buffers(layer):
    c = layer.cfg
    b = {"idx": layer.idx, "w": layer.w, "s_sel": layer.s_sel, "counts": layer.counts,
         "offsets": layer.offsets, "pos": layer.pos, "src": layer.src, "xp": layer.xp,
         "gu": layer.gu, "h": layer.h, "y": layer.y, "out": layer.out}
    if c.router_proj:
        b["logits"] = layer.logits
    if c.S:
        b.update(ys=layer.ys, hs=layer.hs, gus=layer.gus)
    return b


def _pair(wl, backward=True):
    inp = wk.make_inputs(wl, device="cuda")
    cfg = LayerCfg.from_workload(wl)
    step = MoELayer(cfg, inp, "cuda", backward=backward)
    fused = MoELayer(cfg, inp, "cuda", backward=backward)
    return inp, step, fused


def _assert_identical(step, fused):
    assert moe.layer_forward_error(fused.fused, fused.fused_ws) == 0
    a, b = _buffers(step), _buffers(fused)
    for name in a:
        if a[name] is None:
            continue
        assert torch.equal(a[name].view(torch.uint8) if a[name].dtype == torch.bfloat16
                           else a[name], b[name].view(torch.uint8)
                           if b[name].dtype == torch.bfloat16 else b[name]), name


@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_matches_steps_and_oracle(name):
    wl = _wl(REDUCED[name])
    print(f"  case {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.S}", flush=True)
    inp, step, fused = _pair(wl)
    step.forward()
    fused.forward_fused()
    torch.cuda.synchronize()
    _assert_identical(step, fused)
    p = oracle_params(wl, inp)
    r = orc.layer_forward(p)
    assert np.array_equal(host(fused.idx), r["idx"])
    assert np.array_equal(host(fused.offsets), r["offsets"])
    assert np.array_equal(host(fused.pos), r["pos"])
    assert_close(bf(fused.out), r["out"], TOL_BF16, "out")


@pytest.mark.parametrize("name", list(FULL))
def test_fused_full_size_bit_identical(name):
    wl = _wl(FULL[name])
    print(f"  case {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.S}", flush=True)
    inp, step, fused = _pair(wl, backward=False)
    step.forward()
    fused.forward_fused()
    torch.cuda.synchronize()
    _assert_identical(step, fused)
    # repeated single launches give the same bits
    d0 = digest(fused.out, fused.y, fused.h)
    fused.forward_fused()
    torch.cuda.synchronize()
    assert moe.layer_forward_error(fused.fused, fused.fused_ws) == 0
    assert digest(fused.out, fused.y, fused.h) == d0


def test_backward_after_fused_forward():
    """The saves of the single launch drive the backward exactly as the per-step forward's."""
    wl = _wl(REDUCED["mid_t2048"])
    inp, step, fused = _pair(wl)
    step.forward()
    step.backward()
    fused.forward_fused()
    fused.backward()
    torch.cuda.synchronize()
    for name in ("dx", "dw1", "dw2", "dws1", "dws2", "dw_route", "dlogits"):
        assert torch.equal(getattr(step, name), getattr(fused, name)), name


def test_fused_bias_feedback():
    """Sigmoid routing with the load-balancing bias: successive single launches select with
    the bias the previous step's loads produced, as the per-step forward does."""
    wl = _wl(REDUCED["dsv3_e256_zipf"])
    inp = wk.make_inputs(wl, device="cuda")
    cfg = LayerCfg.from_workload(wl)
    cfg.bias_gamma = 0.05
    step = MoELayer(cfg, inp, "cuda", backward=False)
    fused = MoELayer(cfg, inp, "cuda", backward=False)
    for s in range(3):
        step.forward()
        fused.forward_fused()
        torch.cuda.synchronize()
        assert torch.equal(step.idx, fused.idx), s
        assert torch.equal(step.sel_bias, fused.sel_bias), s
        assert torch.equal(step.out.view(torch.uint8), fused.out.view(torch.uint8)), s
