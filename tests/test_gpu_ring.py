"""The macrobatch ring (tokens streamed in minibatches through D ring slots per pass) on the
GPU: every routed row is processed exactly once, the forward and the token-level gradients
are bit-identical to the unstreamed layer for every ring depth D, the weight gradients (reduced
over the passes in pass order) match the oracle, and reruns are bit-identical."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wk
from gpu_harness import TOL_BF16, assert_close, bf, digest, host, oracle_params
from mixture_experts_layer_39_amd.layer import LayerCfg, MoELayer

pytestmark = pytest.mark.gpu

REDUCED = dict(T=512, H=512, E=64, I=256, Is=256)


def _layers(wl, mb, depths, inp=None):
    inp = inp if inp is not None else wk.make_inputs(wl, device="cuda")
    cfg = LayerCfg.from_workload(wl)
    base = MoELayer(cfg, inp, "cuda", backward=True)
    rings = {D: MoELayer(cfg, inp, "cuda", backward=True, minibatch=mb, ring_depth=D)
             for D in depths}
    return inp, base, rings


def _run(layer):
    layer.forward()
    layer.backward()


def _check_conservation(wl, ring):
    k = ring.kr
    counts = host(ring.counts)
    assert counts.sum() == wl.T * k  # every routed row of every minibatch, once
    for p in range(ring.passes):
        t0 = p * ring.pass_tokens
        Tp = min(ring.pass_tokens, wl.T - t0)
        src = host(ring.src[p])[: Tp * k]
        assert np.array_equal(np.sort(src), np.arange(Tp * k))  # a bijection onto the slots
        pos = host(ring.pos[t0:t0 + Tp]).reshape(-1)
        assert np.array_equal(src[pos], np.arange(Tp * k))


@pytest.mark.parametrize("depth", [1, 2, 3, 8])
def test_ring_matches_unstreamed_layer(depth):
    wl = wk.WORKLOADS["dsv3_e256_zipf"].scaled(**REDUCED)
    inp, base, rings = _layers(wl, 64, [depth])
    ring = rings[depth]
    print(f"    D={depth}: {ring.passes} passes of {ring.pass_tokens} tokens", flush=True)
    _run(base)
    _run(ring)
    torch.cuda.synchronize()
    _check_conservation(wl, ring)
    for name in ("idx", "w", "s_sel", "out", "dx", "dw_route", "dlogits", "dws1", "dws2"):
        assert digest(getattr(ring, name)) == digest(getattr(base, name)), name
    # weight gradients sum the same rows in pass order: equal up to rounding
    for name in ("dw1", "dw2"):
        assert_close(bf(getattr(ring, name)), bf(getattr(base, name)), TOL_BF16, name)
    if ring.passes == 1:
        assert digest(ring.dw1, ring.dw2) == digest(base.dw1, base.dw2)


def test_ring_against_oracle():
    wl = wk.WORKLOADS["dsv3_e256_zipf"].scaled(**REDUCED)
    inp, _, rings = _layers(wl, 64, [2])
    ring = rings[2]
    _run(ring)
    torch.cuda.synchronize()
    p = oracle_params(wl, inp)
    r = orc.layer_forward(p)
    g = orc.layer_backward(p, r, wk.bf16_bits(inp["dout"]))
    assert np.array_equal(host(ring.idx), r["idx"])
    assert_close(bf(ring.out), r["out"], TOL_BF16, "out")
    for name in ("dx", "dw1", "dw2", "dws1", "dws2"):
        assert_close(bf(getattr(ring, name)), g[name], TOL_BF16, name)
    assert_close(host(ring.dlogits), g["dlogits"], TOL_BF16, "dlogits")


def test_ring_full_size_bit_identical_to_unstreamed():
    wl = wk.WORKLOADS["dsv3_e256_zipf"]
    inp, base, rings = _layers(wl, wl.minibatch, [2, 4, 16])
    _run(base)
    torch.cuda.synchronize()
    rs = np.random.default_rng(3)
    sample = rs.choice(wl.E, 3, replace=False)
    for D, ring in rings.items():   # 8 passes, 4 passes, one pass over the 16 minibatches
        print(f"    ring depth {D}: {ring.passes} passes", flush=True)
        _run(ring)
        torch.cuda.synchronize()
        _check_conservation(wl, ring)
        for name in ("out", "dx", "dlogits"):
            assert digest(getattr(ring, name)) == digest(getattr(base, name)), (D, name)
        for e in sample:
            assert_close(bf(ring.dw1[e]), bf(base.dw1[e]), TOL_BF16, f"D={D} dw1[{e}]")
            assert_close(bf(ring.dw2[e]), bf(base.dw2[e]), TOL_BF16, f"D={D} dw2[{e}]")
    ring = rings[4]
    hashes = set()
    for _ in range(2):
        _run(ring)
        torch.cuda.synchronize()
        hashes.add(digest(ring.out, ring.dx, ring.dw1, ring.dw2, ring.dws1, ring.dws2))
    assert len(hashes) == 1


def test_forward_only_ring_reuses_one_region():
    wl = wk.WORKLOADS["dsv3_e256_zipf"].scaled(**REDUCED, backward=False)
    inp = wk.make_inputs(wl, device="cuda")
    cfg = LayerCfg.from_workload(wl)
    base = MoELayer(cfg, inp, "cuda", backward=False)
    ring = MoELayer(cfg, inp, "cuda", backward=False, minibatch=64, ring_depth=2)
    assert ring.R == ring.pass_rows  # one ring region of D slots
    base.forward()
    ring.forward()
    torch.cuda.synchronize()
    assert digest(ring.out) == digest(base.out)
