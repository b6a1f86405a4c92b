"""Whole-layer parity (forward and backward) of the HIP path against the CPU oracle.

Reduced sizes (several tiles, ragged tails, empty experts) are compared element by element
against the complete oracle.  The full workload sizes are compared on sampled outputs the
oracle computes one by one: every routing output in full (bit-exact), the layer output, dX,
the routing-weight and logit gradients of sampled tokens, and the weight gradients of sampled
intermediate channels of sampled experts (SwiGLU channels are independent, so a slice of the
weights gives those gradient rows/columns exactly).
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wk
from mixture_experts_layer_39_amd.layer import LayerCfg, MoELayer
from gpu_harness import (TOL_BF16, TOL_MX, assert_close, bf, build_layer, digest, host,
                         layer_outputs, oracle_params)

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny_t128": dict(),
    "mid_t2048": dict(T=384, H=1024, E=8, I=384, Is=256),
    "dsv3_ep64": dict(T=256, H=1024, I=512, R_share=2048),
    "dsv3_ep64_mxfp8": dict(T=256, H=1024, I=512, R_share=2048),
    "dsv3_e256_zipf": dict(T=512, H=512, E=64, I=256, Is=256),
}


def _check_routing(wl, inp, layer, p):
    L = p["logits"] if "logits" in p else orc.router_logits(p["x"], p["w_router"])
    if "w_router" in p:
        assert np.array_equal(host(layer.logits).view(np.uint32), L.view(np.uint32))
    idx, s_sel = orc.route_select(L, wl.k, wl.score, wl.n_groups, wl.topk_groups)
    assert np.array_equal(host(layer.idx), idx)
    assert np.array_equal(host(layer.s_sel).view(np.uint32), s_sel.view(np.uint32))
    w = orc.route_weights(L.astype(np.float64), idx, wl.score, wl.renorm, wl.route_scale)
    assert np.abs(host(layer.w) - w).max() <= 4e-6
    lidx = p.get("idx_local", idx)
    counts, offsets, pos, src = orc.permute(lidx, wl.E)
    assert np.array_equal(host(layer.counts), counts)
    assert np.array_equal(host(layer.offsets), offsets)
    assert np.array_equal(host(layer.pos), pos)
    assert np.array_equal(host(layer.src), src)
    return L, idx, w, lidx, offsets, pos, src


@pytest.mark.parametrize("name", list(REDUCED))
def test_layer_reduced_full_oracle(name):
    wl = wk.WORKLOADS[name].scaled(**REDUCED[name])
    inp, layer = build_layer(wl)
    layer.forward()
    if wl.backward:
        layer.backward()
    torch.cuda.synchronize()
    p = oracle_params(wl, inp)
    _check_routing(wl, inp, layer, p)
    r = orc.layer_forward(p)
    tol = TOL_MX if wl.mx else TOL_BF16
    assert_close(bf(layer.y), r["y"], tol, "y")
    assert_close(bf(layer.out), r["out"], tol, "out")
    if wl.backward:
        g = orc.layer_backward(p, r, wk.bf16_bits(inp["dout"]))
        assert_close(host(layer.dw_route), g["dw_route"], TOL_BF16, "dw_route")
        assert_close(host(layer.dlogits), g["dlogits"], TOL_BF16, "dlogits")
        assert_close(bf(layer.dw2), g["dw2"], TOL_BF16, "dw2")
        assert_close(bf(layer.dw1), g["dw1"], TOL_BF16, "dw1")
        assert_close(bf(layer.dx), g["dx"], TOL_BF16, "dx")
        if wl.S:
            assert_close(bf(layer.dws2), g["dws2"], TOL_BF16, "dws2")
            assert_close(bf(layer.dws1), g["dws1"], TOL_BF16, "dws1")
        # experts that received no rows have exactly zero weight gradients
        for e in np.nonzero(r["counts"] == 0)[0]:
            assert not torch.any(layer.dw1[e] != 0) and not torch.any(layer.dw2[e] != 0)


def test_layer_weight_gradient_tails():
    """Weight gradients of experts with few rows: odd tile counts (45 tiles of dW1, 30 of dW2),
    ragged M and N tails, an expert with no rows between experts with rows, and experts of one
    K step and of several -- against the complete oracle."""
    wl = wk.WORKLOADS["mid_t2048"].scaled(T=160, H=768, E=5, k=2, I=320, S=1, Is=192)
    inp = wk.make_inputs(wl, device="cuda")
    inp["logits"][:, 2] = -30.0   # expert 2 is never among the top 2
    inp["logits"][:, 0] += 2.0    # expert 0 takes most tokens (several K steps)
    layer = MoELayer(LayerCfg.from_workload(wl), inp, "cuda", backward=True)
    print(f"weight-gradient tails case T={wl.T} H={wl.H} E={wl.E} I={wl.I}", flush=True)
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    p = oracle_params(wl, inp)
    r = orc.layer_forward(p)
    counts = r["counts"]
    assert counts[2] == 0 and counts.max() > 128 and counts[counts > 0].min() <= 64, counts
    assert np.array_equal(host(layer.counts), counts)
    g = orc.layer_backward(p, r, wk.bf16_bits(inp["dout"]))
    assert_close(bf(layer.dw1), g["dw1"], TOL_BF16, "dw1")
    assert_close(bf(layer.dw2), g["dw2"], TOL_BF16, "dw2")
    assert_close(bf(layer.dx), g["dx"], TOL_BF16, "dx")
    assert_close(bf(layer.dws1), g["dws1"], TOL_BF16, "dws1")
    assert_close(bf(layer.dws2), g["dws2"], TOL_BF16, "dws2")
    assert not torch.any(layer.dw1[2] != 0) and not torch.any(layer.dw2[2] != 0)


def test_layer_tile_height_boundaries():
    """Experts of exactly 64, 65, 128, 129, 257 and 261 rows: each expert's last M tile sits
    at a boundary of the 64-, 128- and 256-row tile heights (the forward runs tails of at most
    64 rows in the deep ring, the eight-wave backward runs them as 128-row tiles) -- forward
    and backward against the complete oracle.  The share's k = 8 rows per token: 113 tokens."""
    counts = np.array([64, 65, 128, 129, 257, 261])
    T = int(counts.sum()) // 8
    wl = wk.WORKLOADS["dsv3_ep64"].scaled(T=T, H=512, I=256, E=len(counts),
                                          R_share=int(counts.sum()))
    inp = wk.make_inputs(wl, device="cuda")
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(5).shuffle(ids)
    inp["idx_local"] = torch.from_numpy(ids.reshape(T, -1)).to("cuda")
    layer = MoELayer(LayerCfg.from_workload(wl), inp, "cuda", backward=True)
    print(f"tile height boundaries case counts={counts.tolist()}", flush=True)
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    p = oracle_params(wl, inp)
    r = orc.layer_forward(p)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(host(layer.counts), counts)
    assert_close(bf(layer.out), r["out"], TOL_BF16, "out")
    g = orc.layer_backward(p, r, wk.bf16_bits(inp["dout"]))
    for name in ("dx", "dw1", "dw2"):
        assert_close(bf(getattr(layer, name)), g[name], TOL_BF16, name)


def test_layer_tiny_dimensions_full_oracle():
    """H = I = 64 (the smallest the boundary takes): every product a K loop of one or two
    steps, tiles far wider than the operands, weight gradients of 64 x 128 and 128 x 64 --
    forward and backward against the complete oracle."""
    wl = wk.WORKLOADS["mid_t2048"].scaled(T=48, H=64, E=4, k=2, I=64, S=1, Is=64)
    inp = wk.make_inputs(wl, device="cuda")
    layer = MoELayer(LayerCfg.from_workload(wl), inp, "cuda", backward=True)
    print(f"tiny dimensions case T={wl.T} H={wl.H} E={wl.E} I={wl.I}", flush=True)
    layer.forward()
    layer.backward()
    torch.cuda.synchronize()
    p = oracle_params(wl, inp)
    r = orc.layer_forward(p)
    assert np.array_equal(host(layer.counts), r["counts"])
    assert_close(bf(layer.out), r["out"], TOL_BF16, "out")
    g = orc.layer_backward(p, r, wk.bf16_bits(inp["dout"]))
    for name in ("dx", "dw1", "dw2", "dws1", "dws2"):
        assert_close(bf(getattr(layer, name)), g[name], TOL_BF16, name)
    assert_close(host(layer.dlogits), g["dlogits"], TOL_BF16, "dlogits")


def _sampled_forward_backward(wl, inp, layer, p, L, idx, w, lidx, offsets, pos, src, ts, exps,
                              chans):
    k = lidx.shape[1]
    x = orc.bf16_to_f64(p["x"][ts])
    w1b, w2b = inp["w1"], inp["w2"]
    tol = TOL_MX if wl.mx else TOL_BF16
    dq = (lambda a: orc.mx_dequantize(*orc.mx_quantize(a))) if wl.mx else (lambda a: a)
    # forward (and dX) of the sampled tokens
    xq = dq(x)
    yref = np.zeros((len(ts), k, wl.H))
    dxp = np.zeros((len(ts), k, wl.H))
    dout = orc.bf16_to_f64(wk.bf16_bits(inp["dout"][torch.from_numpy(ts).cuda()])) if wl.backward else None
    for e in np.unique(lidx[ts]):
        sel = np.argwhere(lidx[ts] == e)
        w1e = dq(bf(w1b[e:e + 1]))
        w2e = dq(bf(w2b[e:e + 1]))
        xs_ = xq[sel[:, 0]]
        ye, _, _ = orc.ffn_fwd(xs_, np.array([0, len(sel)], np.int32), w1e, w2e, h_mx=wl.mx)
        yref[sel[:, 0], sel[:, 1]] = ye
        if wl.backward:
            dy = w[ts][sel[:, 0], sel[:, 1]][:, None] * dout[sel[:, 0]]
            dxe, _, _ = orc.ffn_bwd(xs_, np.array([0, len(sel)], np.int32), w1e, w2e, dy)
            dxp[sel[:, 0], sel[:, 1]] = dxe
    out = (w[ts][:, :, None] * yref).sum(1)
    dx = dxp.sum(1)
    if wl.S:
        ws1, ws2 = bf(inp["ws1"]), bf(inp["ws2"])
        ys, _, _ = orc.ffn_fwd(x, None, ws1, ws2)
        out = out + ys.sum(0)
        if wl.backward:
            dys = np.broadcast_to(dout, (wl.S,) + dout.shape).reshape(-1, wl.H)
            dxs, _, _ = orc.ffn_bwd(x, None, ws1, ws2, dys)
            dx = dx + dxs.sum(0)
    tsd = torch.from_numpy(ts).cuda()
    assert_close(bf(layer.out[tsd]), out, tol, "out[sampled tokens]")
    if not wl.backward:
        return
    assert_close(bf(layer.dx[tsd]), dx, TOL_BF16, "dx[sampled tokens]")
    dwr = np.einsum("tc,tjc->tj", dout, yref)
    assert_close(host(layer.dw_route)[ts], dwr, TOL_BF16, "dw_route[sampled]")
    dL = orc.router_bwd(L[ts].astype(np.float64), idx[ts], dwr, wl.score, wl.renorm,
                        wl.route_scale)
    assert_close(host(layer.dlogits)[ts], dL, TOL_BF16, "dlogits[sampled]")
    # weight gradients of sampled channels of sampled experts
    xall = None
    doutall = orc.bf16_to_f64(wk.bf16_bits(inp["dout"]))
    xall = orc.bf16_to_f64(p["x"])
    I = wl.I
    ch = np.asarray(chans)
    rows_w1 = np.concatenate([ch, I + ch])
    for e in exps:
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            assert not torch.any(layer.dw1[e] != 0)
            continue
        pr = src[a:b]
        tt, jj = pr // k, pr % k
        xe = xall[tt]
        dy = w[tt, jj][:, None] * doutall[tt]
        w1s = bf(w1b[e][torch.from_numpy(rows_w1).cuda()])[None]
        w2s = bf(w2b[e][:, torch.from_numpy(ch).cuda()])[None]
        _, d1, d2 = orc.ffn_bwd(xe, np.array([0, b - a], np.int32), w1s, w2s, dy)
        assert_close(bf(layer.dw1[e][torch.from_numpy(rows_w1).cuda()]), d1[0], TOL_BF16,
                     f"dw1[e={e}, sampled channels]")
        assert_close(bf(layer.dw2[e][:, torch.from_numpy(ch).cuda()]), d2[0], TOL_BF16,
                     f"dw2[e={e}, sampled channels]")
    if wl.S:
        ws1b, ws2b = inp["ws1"], inp["ws2"]
        chs = ch[ch < wl.Is]
        rs1 = np.concatenate([chs, wl.Is + chs])
        for s in range(wl.S):
            w1s = bf(ws1b[s][torch.from_numpy(rs1).cuda()])[None]
            w2s = bf(ws2b[s][:, torch.from_numpy(chs).cuda()])[None]
            _, d1, d2 = orc.ffn_bwd(xall, np.array([0, wl.T], np.int32), w1s, w2s, doutall)
            assert_close(bf(layer.dws1[s][torch.from_numpy(rs1).cuda()]), d1[0], TOL_BF16,
                         f"dws1[{s}, sampled]")
            assert_close(bf(layer.dws2[s][:, torch.from_numpy(chs).cuda()]), d2[0], TOL_BF16,
                         f"dws2[{s}, sampled]")


@pytest.mark.parametrize("name", ["tiny_t128", "mid_t2048", "dsv3_ep64", "dsv3_ep64_mxfp8",
                                  "dsv3_e256_zipf"])
def test_layer_full_size_sampled(name):
    wl = wk.WORKLOADS[name]
    inp, layer = build_layer(wl)
    layer.forward()
    if wl.backward:
        layer.backward()
    torch.cuda.synchronize()
    p = oracle_params(wl, inp, weights=False)
    L, idx, w, lidx, offsets, pos, src = _check_routing(wl, inp, layer, p)
    counts = np.diff(offsets)
    print(f"    loads: min={counts.min()} median={int(np.median(counts))} max={counts.max()}",
          flush=True)
    rs = np.random.default_rng(7)
    ts = np.sort(rs.choice(wl.T, size=min(wl.T, 6), replace=False))
    nz = np.nonzero(counts)[0]
    exps = sorted({int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])]),
                   int(nz[len(nz) // 2])})
    chans = np.sort(rs.choice(wl.I, size=6, replace=False))
    _sampled_forward_backward(wl, inp, layer, p, L, idx, w, lidx, offsets, pos, src, ts, exps,
                              chans)


@pytest.mark.parametrize("name", ["tiny_t128", "mid_t2048", "dsv3_ep64", "dsv3_ep64_mxfp8"])
def test_layer_bit_identical_reruns(name):
    wl = wk.WORKLOADS[name]
    inp, layer = build_layer(wl)
    hashes = []
    for run in range(3):
        # every output starts from a different byte pattern, so that a value a run does not
        # write itself cannot pass for a reproduced one
        for t in layer_outputs(layer).values():
            t.view(torch.uint8).fill_((0x00, 0x5A, 0xC3)[run])
        layer.forward()
        if wl.backward:
            layer.backward()
        torch.cuda.synchronize()
        hashes.append(digest(*layer_outputs(layer).values()))
    assert hashes[0] == hashes[1] == hashes[2]
