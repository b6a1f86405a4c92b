"""Pins of the oracle's routing against mathematics and brute force (CPU only)."""
import math

import numpy as np
import pytest

import bruteforce as bfc
import workloads as wk


def ulp32(x):
    x = np.abs(np.float32(x))
    return float(np.spacing(x))


def test_rsig_accuracy_and_shape(orc):
    # Dense sweep of [-40, 40]: within 4 ulp of the fp64 logistic function, exact 0.5 at 0,
    # and non-decreasing.
    xs = np.linspace(-40, 40, 40001, dtype=np.float32)
    xs = np.concatenate([xs, np.float32([0.0, -0.0, 1e-30, -1e-30, 0.34657359, 88.0, -88.0])])
    xs = np.sort(xs)
    s = np.array([orc.rsig(x) for x in xs], np.float32)
    ref = 1.0 / (1.0 + np.exp(-np.clip(xs.astype(np.float64), -40, 40)))
    err_ulp = np.abs(s.astype(np.float64) - ref) / np.array([ulp32(r) for r in ref])
    assert err_ulp.max() <= 4.0, err_ulp.max()
    assert orc.rsig(0.0) == np.float32(0.5)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)


def test_router_logits_bit_exact_rules(orc):
    rs = np.random.default_rng(5)
    x = wk.f32_to_bf16_bits(rs.standard_normal((16, 64)).astype(np.float32))
    wr = wk.f32_to_bf16_bits(0.02 * rs.standard_normal((8, 64)).astype(np.float32))
    L = orc.router_logits(x, wr)
    xf, wf = wk.bf16_bits_to_f32(x).astype(np.float64), wk.bf16_bits_to_f32(wr).astype(np.float64)
    exact = xf @ wf.T
    # fp32 sequential sum of exact products: error bounded by H * max partial sum * 2^-24
    bound = 64 * (np.abs(xf) @ np.abs(wf).T) * 2.0 ** -24
    assert np.all(np.abs(L - exact) <= bound)
    # one-hot rows pick a weight exactly
    oh = np.zeros((8, 64), np.uint16)
    for t in range(8):
        oh[t, t * 3] = 0x3F80  # 1.0
    L1 = orc.router_logits(oh, wr)
    for t in range(8):
        assert np.array_equal(L1[t], wk.bf16_bits_to_f32(wr[:, t * 3]))


@pytest.mark.parametrize("score", [wk.SOFTMAX, wk.SIGMOID])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_full_sort(orc, score, ties):
    rs = np.random.default_rng(11 + ties)
    T, E, k = 300, 32, 6
    if ties:
        L = rs.choice(np.float32([-0.5, 0.0, 0.75]), size=(T, E))
    else:
        L = rs.standard_normal((T, E)).astype(np.float32)
    bias = (0.01 * rs.standard_normal(E)).astype(np.float32) if score == wk.SIGMOID else None
    idx, s_sel = orc.route_select(L, k, score, bias=bias)
    if score == wk.SIGMOID:
        keys = np.vectorize(lambda v: orc.rsig(v), otypes=[np.float32])(L)
        keys = (keys + bias[None, :]).astype(np.float32)
    else:
        keys = L
    ref = bfc.topk_by_sort(keys, k)
    assert np.array_equal(idx, ref)
    # selected scores are the sigmoid (without bias) or the logit of the chosen expert
    sel = np.take_along_axis(L, idx, 1)
    if score == wk.SIGMOID:
        assert np.array_equal(s_sel, np.vectorize(lambda v: orc.rsig(v), otypes=[np.float32])(sel))
    else:
        assert np.array_equal(s_sel, sel)
    # distinct experts per token
    assert all(len(set(r)) == k for r in idx)


@pytest.mark.parametrize("ties", [False, True])
def test_group_limited_matches_enumeration(orc, ties):
    rs = np.random.default_rng(3 + ties)
    T, E, k, G, TG = 64, 32, 8, 8, 4
    if ties:
        L = rs.choice(np.float32([-1.0, 0.25, 2.0]), size=(T, E))
    else:
        L = rs.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_select(L, k, wk.SIGMOID, n_groups=G, topk_groups=TG)
    keys = np.vectorize(lambda v: orc.rsig(v), otypes=[np.float32])(L)
    mask = bfc.group_mask_by_enumeration(keys, G, TG, k // TG)
    ref = bfc.topk_by_sort(keys, k, allowed=mask)
    assert np.array_equal(idx, ref)
    # at most topk_groups distinct groups per token
    assert max(len(set((r // (E // G)).tolist())) for r in idx) <= TG


def test_weights_sum_and_restricted_softmax(orc):
    rs = np.random.default_rng(7)
    T, E, k = 200, 16, 4
    L = rs.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_select(L, k, wk.SOFTMAX)
    w = orc.route_weights(L.astype(np.float64), idx, wk.SOFTMAX, True)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    full = np.exp(L.astype(np.float64)) / np.exp(L.astype(np.float64)).sum(1, keepdims=True)
    sel = np.take_along_axis(full, idx, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
    # without renorm: the full softmax at the selected experts
    w_nr = orc.route_weights(L.astype(np.float64), idx, wk.SOFTMAX, False)
    assert np.allclose(w_nr, sel, rtol=1e-13, atol=0)
    # weights are non-increasing along the slots (slot order = key order)
    assert np.all(np.diff(w, axis=1) <= 1e-15)
    # sigmoid with renorm sums to route_scale; without renorm equals route_scale * sigmoid
    idx2, _ = orc.route_select(L, k, wk.SIGMOID)
    ws = orc.route_weights(L.astype(np.float64), idx2, wk.SIGMOID, True, 2.5)
    assert np.allclose(ws.sum(1), 2.5, rtol=1e-14)
    ws_nr = orc.route_weights(L.astype(np.float64), idx2, wk.SIGMOID, False, 2.5)
    sig = 1 / (1 + np.exp(-np.take_along_axis(L.astype(np.float64), idx2, 1)))
    assert np.allclose(ws_nr, 2.5 * sig, rtol=1e-14)


def test_invalid_group_config_rejected(orc):
    L = np.zeros((2, 12), np.float32)
    with pytest.raises(ValueError):
        orc.route_select(L, 4, wk.SIGMOID, n_groups=5, topk_groups=2)  # 12 % 5 != 0
    with pytest.raises(ValueError):
        orc.route_select(L, 13, wk.SOFTMAX)  # k > E
