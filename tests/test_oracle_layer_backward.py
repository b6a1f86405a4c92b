"""Pin of the oracle's whole-layer backward (``oracle.layer_backward``) by central finite
differences of the loss <dout, layer_forward(p)["out"]> (CPU only).

The layer is called exactly as the GPU tests call it -- ``layer_forward`` then
``layer_backward`` on the same parameter dict -- with fp64 values in place of bf16 bits, so
that every composition step of the backward (combine backward, the routed FFN backward, the
shared experts, the un-permute with the shared dX, the router backward with the router's own
expert ids) is checked against the derivative of the forward.  Selection is frozen: the
logits are well separated, so a step of 1e-6 never changes a top-k choice.

Planted slips (monkeypatched into the oracle module, CPU only) must make the check fail: a
dropped shared-expert dX, the local expert ids passed where the router's ids belong, and the
upstream gradient used where the weighted dy belongs.
"""
import numpy as np
import pytest

import workloads as wk

T, H, I, S, Is = 4, 8, 6, 1, 6
STEP = 1e-6
TOL = 1e-6


def _params(score, renorm, n_groups=1, topk_groups=1, local=False, seed=11):
    rs = np.random.default_rng(seed)
    ER = 8
    E = 3 if local else ER
    k = 2
    L = rs.permutation(np.arange(T * ER)).reshape(T, ER).astype(np.float64) * 0.37 - 5.0
    p = dict(x=rs.standard_normal((T, H)), logits=L, k=k, score=score, renorm=renorm,
             route_scale=1.7 if score == wk.SIGMOID else 1.0, n_groups=n_groups,
             topk_groups=topk_groups,
             w1=0.4 * rs.standard_normal((E, 2 * I, H)), w2=0.4 * rs.standard_normal((E, H, I)),
             ws1=0.4 * rs.standard_normal((S, 2 * Is, H)),
             ws2=0.4 * rs.standard_normal((S, H, Is)))
    if local:
        # one GPU's share: the local expert of each routed pair, with a repeated and an
        # empty local expert (E = 3, ids in {0, 2})
        p["idx_local"] = (2 * rs.integers(0, 2, size=(T, k))).astype(np.int32)
    dout = rs.standard_normal((T, H))
    return p, dout


def _grad_errors(orc, p, dout):
    """Relative max error of each analytic gradient of layer_backward against central
    finite differences of the loss."""
    r = orc.layer_forward(p)
    g = orc.layer_backward(p, r, dout)
    idx0 = r["idx"].copy()

    def loss(name, arr):
        q = dict(p)
        q[name] = arr
        rr = orc.layer_forward(q)
        assert np.array_equal(rr["idx"], idx0), "selection moved under the step"
        return float((dout * rr["out"]).sum())

    errs = {}
    for name, gname in [("x", "dx"), ("w1", "dw1"), ("w2", "dw2"), ("ws1", "dws1"),
                        ("ws2", "dws2"), ("logits", "dlogits")]:
        a = p[name]
        num = np.empty_like(a)
        for i in np.ndindex(a.shape):
            a1, a2 = a.copy(), a.copy()
            a1[i] += STEP
            a2[i] -= STEP
            num[i] = (loss(name, a1) - loss(name, a2)) / (2 * STEP)
        errs[gname] = float(np.abs(num - g[gname]).max() / max(np.abs(num).max(), 1e-300))
    return errs


CASES = [
    dict(score=wk.SOFTMAX, renorm=True),
    dict(score=wk.SOFTMAX, renorm=False),
    dict(score=wk.SIGMOID, renorm=True),
    dict(score=wk.SIGMOID, renorm=False),
    dict(score=wk.SIGMOID, renorm=True, n_groups=4, topk_groups=2),
    dict(score=wk.SOFTMAX, renorm=True, local=True),
    dict(score=wk.SIGMOID, renorm=True, local=True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_layer_backward_matches_finite_differences(orc, case):
    p, dout = _params(**case)
    errs = _grad_errors(orc, p, dout)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs


def test_layer_backward_takes_bf16_bits_like_fp64(orc):
    # the GPU tests pass bf16 bit patterns: the same values as fp64 give the same gradients
    p, dout = _params(wk.SIGMOID, True, local=True)
    pb = dict(p)
    for name in ("x", "w1", "w2", "ws1", "ws2"):
        bits = wk.f32_to_bf16_bits(p[name].astype(np.float32))
        pb[name] = bits
        p[name] = orc.bf16_to_f64(bits)
    dbits = wk.f32_to_bf16_bits(dout.astype(np.float32))
    ga = orc.layer_backward(p, orc.layer_forward(p), orc.bf16_to_f64(dbits))
    gb = orc.layer_backward(pb, orc.layer_forward(pb), dbits)
    for key in ga:
        assert np.array_equal(ga[key], gb[key]), key


# ------------------------------------------------------------------ planted slips
def _slip_errors(orc, monkeypatch, case, patch):
    p, dout = _params(**case)
    with monkeypatch.context() as m:
        patch(m, orc, p)
        return _grad_errors(orc, p, dout)


def test_slip_dropped_shared_dx_fails(orc, monkeypatch):
    orig = orc.unpermute

    def patch(m, o, p):
        m.setattr(o, "unpermute", lambda dxp, pos, dxs=None: orig(dxp, pos, None))

    errs = _slip_errors(orc, monkeypatch, dict(score=wk.SOFTMAX, renorm=True), patch)
    assert errs["dx"] > 1e-3, errs


def test_slip_local_ids_in_router_backward_fails(orc, monkeypatch):
    orig = orc.router_bwd

    def patch(m, o, p):
        m.setattr(o, "router_bwd",
                  lambda L, idx, dw, *a: orig(L, p["idx_local"], dw, *a))

    errs = _slip_errors(orc, monkeypatch, dict(score=wk.SIGMOID, renorm=True, local=True),
                        patch)
    assert errs["dlogits"] > 1e-3, errs


def test_slip_dout_for_dy_fails(orc, monkeypatch):
    orig = orc.combine_bwd

    def patch(m, o, p):
        def unweighted(dout, y, pos, w):
            dy, dw = orig(dout, y, pos, np.ones_like(np.asarray(w, np.float64)))
            return dy, orig(dout, y, pos, w)[1]
        m.setattr(o, "combine_bwd", unweighted)

    errs = _slip_errors(orc, monkeypatch, dict(score=wk.SOFTMAX, renorm=True), patch)
    assert errs["dw1"] > 1e-3 and errs["dw2"] > 1e-3 and errs["dx"] > 1e-3, errs
