"""Pins of the oracle's permutation, expert FFN, combine and backward (CPU only)."""
import numpy as np
import pytest

import bruteforce as bfc
import workloads as wk


def test_permutation_matches_stable_argsort(orc):
    rs = np.random.default_rng(1)
    for T, k, E in [(100, 3, 7), (1, 1, 1), (257, 8, 16), (64, 4, 64)]:
        idx = rs.integers(0, E, size=(T, k)).astype(np.int32)
        if E > 3:
            idx[idx == 2] = 1          # force an empty expert
        counts, offsets, pos, src = orc.permute(idx, E)
        c2, o2, p2, s2 = bfc.permutation_by_argsort(idx, E)
        assert np.array_equal(counts, c2) and np.array_equal(offsets, o2)
        assert np.array_equal(pos, p2) and np.array_equal(src, s2)
        # invariants: bijection onto [0, R), src∘pos = id, rows of one expert contiguous
        R = T * k
        assert offsets[-1] == R and counts.sum() == R
        assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(R))
        assert np.array_equal(src[pos.reshape(-1)], np.arange(R))
        e_of_row = np.repeat(np.arange(E), counts)
        assert np.array_equal(e_of_row[pos.reshape(-1)], idx.reshape(-1))
        for e in range(E):
            assert np.all(np.diff(src[offsets[e]:offsets[e + 1]]) > 0)


def test_dispatch_copies_rows(orc):
    rs = np.random.default_rng(2)
    x = rs.integers(0, 65535, size=(10, 16)).astype(np.uint16)
    idx = rs.integers(0, 3, size=(10, 2)).astype(np.int32)
    _, _, pos, src = orc.permute(idx, 3)
    xp = orc.dispatch(x, 2, src)
    for t in range(10):
        for j in range(2):
            assert np.array_equal(xp[pos[t, j]], x[t])


def _rand(rs, *shape, s=1.0):
    return s * rs.standard_normal(shape)


def test_ffn_single_expert_is_dense_swiglu(orc):
    rs = np.random.default_rng(3)
    R, H, I = 9, 24, 10
    x, w1, w2 = _rand(rs, R, H), _rand(rs, 1, 2 * I, H, s=0.3), _rand(rs, 1, H, I, s=0.3)
    y, gu, h = orc.ffn_fwd(x, np.array([0, R], np.int32), w1, w2, want_gu=True, want_h=True)
    ref = bfc.dense_swiglu(x, w1[0], w2[0])
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.allclose(gu[:, :I], x @ w1[0, :I].T, rtol=1e-12)
    # the layer with one expert, k = 1 and renormalised weights is the dense FFN
    idx = np.zeros((R, 1), np.int32)
    _, off, pos, src = orc.permute(idx, 1)
    out = orc.combine(y[src], pos, np.ones((R, 1)))  # y is in expert order = token order
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_ffn_experts_are_independent_blocks(orc):
    # each expert's rows equal the dense FFN of that expert on those rows; empty experts ok
    rs = np.random.default_rng(4)
    H, I = 16, 8
    offsets = np.array([0, 3, 3, 10, 11], np.int32)
    R, E = 11, 4
    x, w1, w2 = _rand(rs, R, H), _rand(rs, E, 2 * I, H, s=0.3), _rand(rs, E, H, I, s=0.3)
    y, _, _ = orc.ffn_fwd(x, offsets, w1, w2)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            assert np.allclose(y[a:b], bfc.dense_swiglu(x[a:b], w1[e], w2[e]), rtol=1e-12)
    # shared mode: every expert takes all rows
    ys, _, _ = orc.ffn_fwd(x, None, w1, w2)
    for e in range(E):
        assert np.allclose(ys[e], bfc.dense_swiglu(x, w1[e], w2[e]), rtol=1e-12)


def test_combine_conservation(orc):
    rs = np.random.default_rng(5)
    T, H, E, k = 40, 12, 6, 3
    L = rs.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_select(L, k, wk.SOFTMAX)
    w = orc.route_weights(L.astype(np.float64), idx, wk.SOFTMAX, True)
    _, _, pos, src = orc.permute(idx, E)
    x = rs.standard_normal((T, H))
    # identity experts (y = dispatched x) with renormalised weights give back x
    y = x[src // k]
    assert np.allclose(orc.combine(y, pos, w), x, rtol=1e-14, atol=1e-14)
    # tag test: y[r,:] = r with k = 1 and unit weight returns pos exactly
    idx1 = idx[:, :1].copy()
    _, _, pos1, _ = orc.permute(idx1, E)
    tag = np.repeat(np.arange(T, dtype=np.float64)[:, None], H, 1)
    out = orc.combine(tag, pos1, np.ones((T, 1)))
    assert np.array_equal(out[:, 0], pos1[:, 0].astype(np.float64))
    # one-hot weights over k slots: every routed row reached exactly once
    R = T * k
    tagk = np.repeat(np.arange(R, dtype=np.float64)[:, None], H, 1)
    seen = []
    for j in range(k):
        oh = np.zeros((T, k))
        oh[:, j] = 1
        seen.append(orc.combine(tagk, pos, oh)[:, 0])
    assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(R, dtype=np.float64))
    # shared experts are added with weight one
    ys = rs.standard_normal((2, T, H))
    assert np.allclose(orc.combine(y, pos, w, ys), x + ys[0] + ys[1], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ finite differences
def _layer_f64(orc, x, w1, w2, ws1, ws2, L, idx, lidx, score, renorm, scale, E):
    k = lidx.shape[1]
    _, offsets, pos, src = orc.permute(lidx, E)
    w = orc.route_weights(L, idx, score, renorm, scale)
    xp = x[src // k]
    y, _, _ = orc.ffn_fwd(xp, offsets, w1, w2)
    ys = orc.ffn_fwd(x, None, ws1, ws2)[0] if ws1 is not None else None
    return orc.combine(y, pos, w, ys)


@pytest.mark.parametrize("score,renorm", [(wk.SOFTMAX, True), (wk.SOFTMAX, False),
                                          (wk.SIGMOID, True), (wk.SIGMOID, False)])
def test_backward_matches_finite_differences(orc, score, renorm):
    rs = np.random.default_rng(6)
    T, H, E, k, I, S, Is = 4, 8, 4, 2, 6, 1, 6
    scale = 1.7
    x = rs.standard_normal((T, H))
    w1, w2 = 0.4 * rs.standard_normal((E, 2 * I, H)), 0.4 * rs.standard_normal((E, H, I))
    ws1, ws2 = 0.4 * rs.standard_normal((S, 2 * Is, H)), 0.4 * rs.standard_normal((S, H, Is))
    # logits with well separated values so the selection stays frozen under the step
    L = rs.permutation(np.arange(T * E)).reshape(T, E).astype(np.float64) * 0.37 - 3.0
    idx, _ = orc.route_select(L.astype(np.float32), k, score)
    lidx = idx % E
    dout = rs.standard_normal((T, H))
    args = dict(score=score, renorm=renorm, scale=scale, E=E)

    def loss(x_=x, w1_=w1, w2_=w2, ws1_=ws1, ws2_=ws2, L_=L):
        return float((dout * _layer_f64(orc, x_, w1_, w2_, ws1_, ws2_, L_, idx, lidx,
                                        **args)).sum())

    # analytic gradients from the oracle's backward
    _, offsets, pos, src = orc.permute(lidx, E)
    w = orc.route_weights(L, idx, score, renorm, scale)
    xp = x[src // k]
    y, _, _ = orc.ffn_fwd(xp, offsets, w1, w2)
    dy, dw = orc.combine_bwd(dout, y, pos, w)
    dxp, dw1, dw2 = orc.ffn_bwd(xp, offsets, w1, w2, dy)
    dys = np.broadcast_to(dout, (S, T, H)).reshape(S * T, H)
    dxs, dws1, dws2 = orc.ffn_bwd(x, None, ws1, ws2, dys)
    dx = orc.unpermute(dxp, pos, dxs)
    dL = orc.router_bwd(L, idx, dw, score, renorm, scale)

    def fd(name, arr, grad):
        h = 1e-6
        num = np.empty_like(arr)
        for i in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[i] += h
            a2[i] -= h
            num[i] = (loss(**{name: a1}) - loss(**{name: a2})) / (2 * h)
        err = np.abs(num - grad).max() / max(np.abs(num).max(), 1e-300)
        assert err <= 1e-6, (name, err)

    fd("x_", x, dx)
    fd("w1_", w1, dw1)
    fd("w2_", w2, dw2)
    fd("ws1_", ws1, dws1)
    fd("ws2_", ws2, dws2)
    fd("L_", L, dL)
