"""The oracle's whole-layer composition, pinned per token against dense products (CPU)."""
import numpy as np
import pytest

import bruteforce as bfc
import workloads as wk


def _params(wl, inp):
    p = dict(x=wk.bf16_bits(inp["x"]), k=wl.k, score=wl.score, renorm=wl.renorm,
             route_scale=wl.route_scale, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
             w1=wk.bf16_bits(inp["w1"]), w2=wk.bf16_bits(inp["w2"]), mx=wl.mx)
    if "w_router" in inp:
        p["w_router"] = wk.bf16_bits(inp["w_router"])
    else:
        p["logits"] = inp["logits"].numpy()
    if "idx_local" in inp:
        p["idx_local"] = inp["idx_local"].numpy()
    if wl.S:
        p["ws1"], p["ws2"] = wk.bf16_bits(inp["ws1"]), wk.bf16_bits(inp["ws2"])
    return p


@pytest.mark.parametrize("name,over", [
    ("tiny_t128", dict(T=24)),
    ("mid_t2048", dict(T=20, H=64, E=8, I=32, Is=32)),
    ("dsv3_ep64", dict(T=16, H=64, I=32, R_share=128)),
    ("dsv3_e256_zipf", dict(T=12, H=64, I=32, Is=32, E=32)),
    ("dsv3_ep64_mxfp8", dict(T=16, H=64, I=64, R_share=128)),
])
def test_layer_forward_per_token(orc, name, over):
    wl = wk.WORKLOADS[name].scaled(**over)
    inp = wk.make_inputs(wl)
    p = _params(wl, inp)
    r = orc.layer_forward(p)
    x = orc.bf16_to_f64(p["x"])
    w1, w2 = orc.bf16_to_f64(p["w1"]), orc.bf16_to_f64(p["w2"])
    lidx = p.get("idx_local", r["idx"])
    if wl.mx:
        x = orc.mx_dequantize(*orc.mx_quantize(x))
        w1 = orc.mx_dequantize(*orc.mx_quantize(w1))
        w2 = orc.mx_dequantize(*orc.mx_quantize(w2))
    ref = np.zeros_like(r["out"])
    for t in range(wl.T):
        for j in range(lidx.shape[1]):
            e = lidx[t, j]
            if wl.mx:
                I = w1.shape[1] // 2
                g = x[t] @ w1[e, :I].T
                u = x[t] @ w1[e, I:].T
                h = orc.mx_dequantize(*orc.mx_quantize((g / (1 + np.exp(-g)) * u)[None]))[0]
                yv = h @ w2[e].T
            else:
                yv = bfc.dense_swiglu(x[t][None], w1[e], w2[e])[0]
            ref[t] += r["w"][t, j] * yv
        for s in range(wl.S):
            ws1, ws2 = orc.bf16_to_f64(p["ws1"]), orc.bf16_to_f64(p["ws2"])
            ref[t] += bfc.dense_swiglu(x[t][None], ws1[s], ws2[s])[0]
    assert np.allclose(r["out"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())
    if wl.local_share:
        assert np.array_equal(r["counts"], inp["counts_local"].numpy())


def test_workload_generators_are_seeded():
    wl = wk.WORKLOADS["dsv3_e256_zipf"].scaled(T=64, H=64, I=32, Is=32)
    a, b = wk.make_inputs(wl), wk.make_inputs(wl)
    for key in a:
        assert np.array_equal(np.asarray(a[key].float() if a[key].dtype == wk.torch.bfloat16
                                         else a[key]),
                              np.asarray(b[key].float() if b[key].dtype == wk.torch.bfloat16
                                         else b[key]))
    # Zipf logits: top-1 expert frequencies follow the popularity ranking
    wl2 = wk.WORKLOADS["dsv3_e256_zipf"].scaled(T=20000)
    L = wk.router_logits(wl2)
    top1 = np.bincount(L.argmax(1), minlength=256)
    assert top1.max() > 0.15 * wl2.T


def test_local_share_counts():
    wl = wk.WORKLOADS["dsv3_ep64"]
    li, c = wk.local_share_idx(wl)
    assert li.shape == (2048, 8) and c.sum() == 16384
    assert np.array_equal(np.bincount(li.reshape(-1), minlength=4), c)
