"""Pins of the oracle's backward with MXFP8 dgrad products (ffn_bwd_mx), CPU only.

What fixes it without re-running its own formula:
- lossless operands: when dy is exactly MX-representable along H and W2 / W1 along their
  contraction dimensions (pre-quantised), every quantisation before dGU is the identity, so
  dGU and both weight gradients equal the BF16 oracle's (itself pinned by finite
  differences), and dXp differs from it only by one E4M3 rounding of dGU.  Values k/8 with
  integer |k| <= 8 are exact in E4M3 under any block scale, so dy and h drawn from them make
  the token-axis quantisation of dW2's operands the identity too;
- power-of-two equivariance: MX quantisation along a dimension commutes with scaling a whole
  line along that dimension by 2^s (the block scale moves, the codes do not).  Scaling a row
  of dy, a column of W1 or a column of W2 must therefore scale the matching output lines by
  exactly 2^s; a quantisation along the wrong dimension would mix differently scaled values
  in one block and break the equality.  For the token-axis (weight-gradient) quantisation a
  whole channel column of xp scales dW1's column, and a W2 column scales dGU's channel and
  with it dW1's rows.
"""
import numpy as np

RS = np.random.default_rng(7)


def _case(E=3, H=64, I=64, counts=(40, 0, 37)):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    xp = RS.normal(size=(R, H))
    w1 = RS.normal(size=(E, 2 * I, H)) * 0.1
    w2 = RS.normal(size=(E, H, I)) * 0.1
    dy = RS.normal(size=(R, H))
    gu = RS.normal(size=(R, 2 * I)) * 2
    h = RS.normal(size=(R, I))
    return off, xp, w1, w2, dy, gu, h


def _pre_rows(orc, a):        # exactly MX-representable along the last dimension
    return orc.mx_dequantize(*orc.mx_quantize(a))


def _pre_cols(orc, w):        # [E, A, B]: exactly representable along A, per column
    return np.stack([_pre_rows(orc, np.ascontiguousarray(m.T)).T for m in w])


def test_lossless_operands_match_bf16_oracle(orc):
    off, xp, w1, w2, dy, gu, h = _case()
    dy = _pre_rows(orc, dy)
    w2 = _pre_cols(orc, w2)
    w1 = _pre_cols(orc, w1)
    # the BF16 oracle differentiates the forward itself: give the MX backward the g|u and h
    # of the same forward
    y, gu_f, h_f = orc.ffn_fwd(xp, off, w1, w2, want_gu=True, want_h=True)
    dxp_m, dgu_m, dw1_m, dw2_m = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu_f, h_f)
    dxp_b, dw1_b, dw2_b = orc.ffn_bwd(xp, off, w1, w2, dy)
    assert np.allclose(dw1_m, dw1_b, rtol=1e-10, atol=1e-10)
    assert np.allclose(dw2_m, dw2_b, rtol=1e-10, atol=1e-10)
    rel = np.linalg.norm(dxp_m - dxp_b) / np.linalg.norm(dxp_b)
    assert 1e-6 < rel < 0.1          # one E4M3 rounding of dGU, and not exact
    # an expert with no rows has zero weight gradients
    assert not dw1_m[1].any() and not dw2_m[1].any()


def test_dy_rows_equivariant(orc):
    off, xp, w1, w2, dy, gu, h = _case()
    s = RS.integers(-3, 4, size=dy.shape[0]).astype(np.float64)
    a = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h)
    b = orc.ffn_bwd_mx(xp, off, w1, w2, dy * 2.0 ** s[:, None], gu, h)
    assert np.array_equal(b[0], a[0] * 2.0 ** s[:, None])      # dXp rows
    assert np.array_equal(b[1], a[1] * 2.0 ** s[:, None])      # dGU rows


def test_w1_columns_equivariant(orc):
    off, xp, w1, w2, dy, gu, h = _case()
    s = RS.integers(-3, 4, size=w1.shape[2]).astype(np.float64)
    a = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h)
    b = orc.ffn_bwd_mx(xp, off, w1 * 2.0 ** s[None, None, :], w2, dy, gu, h)
    assert np.array_equal(b[0], a[0] * 2.0 ** s[None, :])      # dXp columns


def test_w2_columns_equivariant(orc, mxw=False):
    off, xp, w1, w2, dy, gu, h = _case()
    s = RS.integers(-3, 4, size=w2.shape[2]).astype(np.float64)
    a = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h, mx_wgrad=mxw)
    b = orc.ffn_bwd_mx(xp, off, w1, w2 * 2.0 ** s[None, None, :], dy, gu, h, mx_wgrad=mxw)
    I = w2.shape[2]
    sc = np.concatenate([s, s])
    assert np.array_equal(b[1], a[1] * 2.0 ** sc[None, :])     # dGU channels (gate and up)
    assert np.array_equal(b[2], a[2] * 2.0 ** sc[None, :, None])  # dW1 rows
    assert np.array_equal(b[3], a[3])                          # dW2 does not see W2


def test_w2_columns_equivariant_mx_wgrad(orc):
    test_w2_columns_equivariant(orc, mxw=True)


def test_mx_wgrad_lossless_and_xp_columns(orc):
    off, xp, w1, w2, dy, gu, h = _case(counts=(40, 0, 37))
    k8 = lambda shape: RS.integers(-8, 9, size=shape) / 8.0
    dy, h, xp = k8(dy.shape), k8(h.shape), k8(xp.shape)
    a = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h, mx_wgrad=True)
    b = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h, mx_wgrad=False)
    assert np.array_equal(a[3], b[3])                     # dW2: token-axis quantisation exact
    rel = np.linalg.norm(a[2] - b[2]) / np.linalg.norm(b[2])
    assert 1e-6 < rel < 0.1                               # dW1: dGU quantised along tokens
    # a power-of-two scale per xp column scales dW1's columns exactly
    s = RS.integers(-3, 4, size=xp.shape[1]).astype(np.float64)
    c = orc.ffn_bwd_mx(xp * 2.0 ** s[None, :], off, w1, w2, dy, gu, h, mx_wgrad=True)
    assert np.array_equal(c[2], a[2] * 2.0 ** s[None, None, :])


def test_mx_wgrad_blocks_start_at_the_experts_first_row(orc):
    # expert 0: 40 rows = one full 32-row block and 8 rows in a zero-padded second block.
    # Rows 32..39 are 2^-20 smaller: in a block of their own they keep their precision, in a
    # block shared with rows 8..31 (blocks aligned anywhere else) they would flush to zero.
    off, xp, w1, w2, dy, gu, h = _case(counts=(40, 0, 37))
    xp[32:40] *= 2.0 ** -20
    tiny = xp.copy()
    tiny[:32] = 0.0
    a = orc.ffn_bwd_mx(xp, off, w1, w2, dy, gu, h, mx_wgrad=True)
    b = orc.ffn_bwd_mx(tiny, off, w1, w2, dy, gu, h, mx_wgrad=True)
    big = xp.copy()
    big[32:40] = 0.0
    c = orc.ffn_bwd_mx(big, off, w1, w2, dy, gu, h, mx_wgrad=True)
    # the small rows' share of dW1_0 survives exactly as when they are quantised alone
    assert np.array_equal(a[2][0] - c[2][0], b[2][0])
    assert np.abs(b[2][0]).max() > 0


def test_mx_wgrad_couples_rows_of_a_token_block(orc):
    # doubling one token row of xp (h) changes the block's scale and with it the codes of the
    # other rows of its 32-token block: dW1 (dW2) is no longer the linear update.  Without a
    # token-axis quantisation (none, or along channels) the update would be exactly linear.
    off, xp, w1, w2, dy, gu, h = _case(counts=(64, 0, 37))
    for name, arr, out in (("xp", xp, 2), ("h", h, 3)):
        r = int(np.argmax(np.abs(arr[:32]).max(axis=1)))      # the row holding a block max
        two = arr.copy()
        two[r] *= 2.0
        kw = dict(xp=xp, h=h)
        kw[name] = arr
        a = orc.ffn_bwd_mx(kw["xp"], off, w1, w2, dy, gu, kw["h"], mx_wgrad=True)
        kw[name] = two
        b = orc.ffn_bwd_mx(kw["xp"], off, w1, w2, dy, gu, kw["h"], mx_wgrad=True)
        only = np.zeros_like(arr)
        only[r] = arr[r]
        kw[name] = only
        c = orc.ffn_bwd_mx(kw["xp"], off, w1, w2, dy, gu, kw["h"], mx_wgrad=True)
        assert not np.allclose(b[out][0], a[out][0] + c[out][0], rtol=1e-9, atol=0), name


def test_bf16_round_matches_torch(orc):
    import torch
    a = np.concatenate([RS.normal(size=4000) * 10.0 ** RS.integers(-30, 30, size=4000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875]])
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_round(a), ref)


def test_channel_block_slice_is_exact(orc):
    """The MXFP8 forward and backward of one 32-channel block of an expert, computed from the
    sliced weights alone, equal that block of the full-width computation bit for bit: h is
    quantised along I in blocks of 32, W1 rows and W2^T rows along H, and the weight-gradient
    operands along the tokens column by column, so no MX block crosses the slice.  (The GPU
    test of the full-size MXFP8 backward samples weight gradients this way.)"""
    rs = np.random.default_rng(0)
    M, H, I = 150, 256, 128
    xe = orc.bf16_round(rs.standard_normal((M, H)))
    w1 = orc.bf16_round(rs.standard_normal((1, 2 * I, H)) * 0.05)
    w2 = orc.bf16_round(rs.standard_normal((1, H, I)) * 0.05)
    dy = rs.standard_normal((M, H))
    dq = lambda a: orc.mx_dequantize(*orc.mx_quantize(a))
    xq, off = dq(xe), np.array([0, M], np.int32)
    _, gu, h = orc.ffn_fwd(xq, off, dq(w1), dq(w2), h_mx=True, want_gu=True, want_h=True)
    _, _, dw1, dw2 = orc.ffn_bwd_mx(xq, off, w1, w2, dy, gu, h, mx_wgrad=True)
    ch = np.arange(64, 96)
    rows = np.concatenate([ch, I + ch])
    w1s, w2s = w1[:, rows], w2[:, :, ch]
    _, gus, hs = orc.ffn_fwd(xq, off, dq(w1s), dq(w2s), h_mx=True, want_gu=True, want_h=True)
    assert np.array_equal(hs, h[:, ch]) and np.array_equal(gus, gu[:, rows])
    _, _, dw1s, dw2s = orc.ffn_bwd_mx(xq, off, w1s, w2s, dy, gus, hs, mx_wgrad=True)
    assert np.array_equal(dw1s[0], dw1[0][rows]) and np.array_equal(dw2s[0], dw2[0][:, ch])
