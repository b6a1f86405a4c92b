"""Per-call parity of the HIP path against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wk
import mixture_experts_layer_39_amd as moe
from gpu_harness import TOL_BF16, TOL_MX, assert_close, bf, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _route_gpu(logits, T, E, k, score, n_groups=1, topk_groups=1, renorm=True, scale=1.0,
               bias=None, x=None, wr=None, H=0):
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(idx=torch.empty(T, k, **i32), w=torch.empty(T, k, device=DEV),
               s_sel=torch.empty(T, k, device=DEV), counts=torch.empty(E, **i32),
               offsets=torch.empty(E + 1, **i32), pos=torch.empty(T, k, **i32),
               src=torch.empty(max(T * k, 1), **i32))
    ws = torch.empty(max(moe.route_workspace_size(T, k, E), 256), dtype=torch.uint8, device=DEV)
    moe.moe_route(logits, T, E, k, x=x, w_router=wr, H=H, score=score, n_groups=n_groups,
                  topk_groups=topk_groups, renorm=renorm, route_scale=scale, sel_bias=bias,
                  ws=ws, **out)
    torch.cuda.synchronize()
    return {kk: host(v) for kk, v in out.items()}


ROUTE_CASES = [
    # name, T, E, k, score, groups, topk_groups, renorm, scale, logits kind
    ("softmax_top2_of_8", 128, 8, 2, wk.SOFTMAX, 1, 1, True, 1.0, "normal"),
    ("softmax_top6_of_64", 2048, 64, 6, wk.SOFTMAX, 1, 1, True, 1.0, "normal"),
    ("softmax_top6_no_renorm", 512, 64, 6, wk.SOFTMAX, 1, 1, False, 1.0, "normal"),
    ("sigmoid_top8_of_256", 2048, 256, 8, wk.SIGMOID, 1, 1, True, 1.0, "normal"),
    ("sigmoid_group8_top4_zipf", 8192, 256, 8, wk.SIGMOID, 8, 4, True, 1.0, "zipf"),
    ("sigmoid_scale2.5_no_renorm", 300, 96, 5, wk.SIGMOID, 1, 1, False, 2.5, "normal"),
    ("softmax_ties", 700, 32, 4, wk.SOFTMAX, 1, 1, True, 1.0, "ties"),
    ("sigmoid_group_ties", 500, 64, 8, wk.SIGMOID, 8, 4, True, 1.0, "ties"),
    ("k_equals_E", 33, 16, 16, wk.SOFTMAX, 1, 1, True, 1.0, "normal"),
    ("one_token", 1, 1024, 8, wk.SIGMOID, 1, 1, True, 1.0, "normal"),
    ("wide_sigmoid_range", 257, 128, 8, wk.SIGMOID, 1, 1, True, 1.0, "wide"),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_parity(case):
    name, T, E, k, score, G, TG, renorm, scale, kind = case
    rs = np.random.default_rng(abs(hash(name)) % 2 ** 32)
    if kind == "zipf":
        L = wk.router_logits(wk.WORKLOADS["dsv3_e256_zipf"].scaled(T=T))
    elif kind == "ties":
        L = rs.choice(np.float32([-0.75, 0.0, 1.5]), size=(T, E))
    elif kind == "wide":
        L = (rs.standard_normal((T, E)) * 30).astype(np.float32)
    else:
        L = rs.standard_normal((T, E)).astype(np.float32)
    bias = None
    if score == wk.SIGMOID and name.startswith("sigmoid_scale"):
        bias = (0.05 * rs.standard_normal(E)).astype(np.float32)
    got = _route_gpu(torch.from_numpy(L).to(DEV), T, E, k, score, G, TG, renorm, scale,
                     None if bias is None else torch.from_numpy(bias).to(DEV))
    idx, s_sel = orc.route_select(L, k, score, G, TG, bias)
    assert np.array_equal(got["idx"], idx)
    assert np.array_equal(got["s_sel"].view(np.uint32), s_sel.view(np.uint32))
    w = orc.route_weights(L.astype(np.float64), idx, score, renorm, scale)
    assert np.abs(got["w"] - w).max() <= 4e-6 * max(1.0, scale)
    counts, offsets, pos, src = orc.permute(idx, E)
    for nm, ref in (("counts", counts), ("offsets", offsets), ("pos", pos), ("src", src)):
        assert np.array_equal(got[nm].reshape(ref.shape), ref), nm


def test_router_projection_bit_exact():
    wl = wk.WORKLOADS["tiny_t128"]
    inp = wk.make_inputs(wl, device=DEV, weights=False)
    T, E, H = wl.T, wl.E, wl.H
    logits = torch.empty(T, E, device=DEV)
    got = _route_gpu(logits, T, E, wl.k, wl.score, x=inp["x"], wr=inp["w_router"], H=H)
    ref = orc.router_logits(wk.bf16_bits(inp["x"]), wk.bf16_bits(inp["w_router"]))
    assert np.array_equal(host(logits).view(np.uint32), ref.view(np.uint32))
    idx, _ = orc.route_select(ref, wl.k, wl.score)
    assert np.array_equal(got["idx"], idx)


@pytest.mark.parametrize("kind", ["local_share", "one_expert", "empty_experts", "empty_input"])
def test_route_given_experts(kind):
    if kind == "local_share":
        wl = wk.WORKLOADS["dsv3_ep64"]
        ids, c = wk.local_share_idx(wl)
        E = wl.E
    elif kind == "one_expert":
        ids, E = np.full((1000, 3), 5, np.int32), 7
    elif kind == "empty_experts":
        rs = np.random.default_rng(2)
        ids, E = (rs.integers(0, 4, size=(513, 6)) * 37).astype(np.int32), 256
    else:
        ids, E = np.zeros((0, 4), np.int32), 16
    T, k = ids.shape
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    pos, src = torch.empty(max(T, 1), k, **i32), torch.empty(max(T * k, 1), **i32)
    ws = torch.empty(max(moe.route_workspace_size(T, k, E), 256), dtype=torch.uint8, device=DEV)
    moe.moe_route(None, T, E, k, idx_in=torch.from_numpy(ids).to(DEV), counts=counts,
                  offsets=offsets, pos=pos, src=src, ws=ws)
    torch.cuda.synchronize()
    rc, ro, rp, rsrc = orc.permute(ids, E)
    assert np.array_equal(host(counts), rc) and np.array_equal(host(offsets), ro)
    if T:
        assert np.array_equal(host(pos)[:T], rp) and np.array_equal(host(src)[:T * k], rsrc)
    if kind == "local_share":
        assert np.array_equal(host(counts), c)


def test_dispatch_bit_exact_and_mx():
    rs = np.random.default_rng(3)
    T, H, k = 300, 512, 3
    x = wk.normal_bf16(wk.WORKLOADS["mid_t2048"], "x", 9, (T, H), 1.0, DEV)
    ids = rs.integers(0, 5, size=(T, k)).astype(np.int32)
    _, _, _, src = orc.permute(ids, 5)
    R = T * k
    xp = torch.empty(R, H, dtype=torch.bfloat16, device=DEV)
    moe.moe_dispatch(x, T, H, k, torch.from_numpy(src).to(DEV), R, xp)
    xq = torch.empty(R, H, dtype=torch.uint8, device=DEV)
    xs = torch.empty(R, H // 32, dtype=torch.uint8, device=DEV)
    xp2 = torch.empty_like(xp)
    moe.moe_dispatch(x, T, H, k, torch.from_numpy(src).to(DEV), R, xp2, xq, xs)
    torch.cuda.synchronize()
    ref = orc.dispatch(wk.bf16_bits(x), k, src)
    assert np.array_equal(wk.bf16_bits(xp), ref)
    assert np.array_equal(wk.bf16_bits(xp2), ref)
    # token-driven form (pos): same rows, bit for bit, in both precisions
    pos_ = np.empty(R, dtype=np.int32)
    pos_[src] = np.arange(R, dtype=np.int32)
    pos_d = torch.from_numpy(pos_.reshape(T, k)).to(DEV)
    xp3 = torch.empty_like(xp)
    moe.moe_dispatch(x, T, H, k, None, R, xp3, pos=pos_d)
    xq3, xs3 = torch.empty_like(xq), torch.empty_like(xs)
    moe.moe_dispatch(x, T, H, k, None, R, None, xq3, xs3, pos=pos_d)
    torch.cuda.synchronize()
    assert np.array_equal(wk.bf16_bits(xp3), ref)
    assert torch.equal(xq3, xq) and torch.equal(xs3, xs)
    # token-driven MX form that also writes the bf16 rows
    xp4, xq4, xs4 = torch.empty_like(xp), torch.empty_like(xq), torch.empty_like(xs)
    moe.moe_dispatch(x, T, H, k, None, R, xp4, xq4, xs4, pos=pos_d)
    torch.cuda.synchronize()
    assert np.array_equal(wk.bf16_bits(xp4), ref)
    assert torch.equal(xq4, xq) and torch.equal(xs4, xs)
    cq, cs = orc.mx_quantize(orc.bf16_to_f64(ref))
    assert np.array_equal(host(xq), cq) and np.array_equal(host(xs), cs)


@pytest.mark.parametrize("mode", [moe.MX_FLOOR, moe.MX_CEIL])
def test_mx_quantize_bit_exact(mode):
    # every finite bf16 bit pattern, in shuffled blocks of 32 (wide range per block) and in
    # sorted blocks (neighbouring values: normal codes, and saturation at 448 next to each
    # block maximum in floor mode), plus wide-range fp32 values
    rs = np.random.default_rng(4)
    bits = np.arange(65536, dtype=np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    n = (len(finite) // 32) * 32
    finite = np.concatenate([rs.permutation(finite)[:n], np.sort(finite)[:n]]).reshape(-1, 32 * 8)
    t = torch.from_numpy(finite.view(np.int16)).to(DEV).view(torch.bfloat16)
    rows, K = finite.shape
    q = torch.empty(rows, K, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, K // 32, dtype=torch.uint8, device=DEV)
    moe.mx_quantize(t, moe.BF16, rows, K, q, s, mode)
    f = (rs.standard_normal((64, 256)) * np.exp2(rs.integers(-60, 60, size=(64, 1)))).astype(np.float32)
    f[5, :32] = 0.0
    tf = torch.from_numpy(f).to(DEV)
    qf = torch.empty(64, 256, dtype=torch.uint8, device=DEV)
    sf = torch.empty(64, 8, dtype=torch.uint8, device=DEV)
    moe.mx_quantize(tf, moe.F32, 64, 256, qf, sf, mode)
    torch.cuda.synchronize()
    rq, rsc = orc.mx_quantize(orc.bf16_to_f64(finite), mode)
    assert np.array_equal(host(s), rsc)
    assert np.array_equal(host(q), rq)
    rq2, rs2 = orc.mx_quantize(f.astype(np.float64), mode)
    assert np.array_equal(host(sf), rs2) and np.array_equal(host(qf), rq2)


def test_combine_parity():
    rs = np.random.default_rng(5)
    T, H, k, S, E = 333, 768, 4, 2, 9
    wl = wk.WORKLOADS["mid_t2048"]
    R = T * k
    y = wk.normal_bf16(wl, "x", 11, (R, H), 1.0, DEV)
    ys = wk.normal_bf16(wl, "x", 12, (S, T, H), 1.0, DEV)
    ids = rs.integers(0, E, size=(T, k)).astype(np.int32)
    _, _, pos, _ = orc.permute(ids, E)
    w = rs.random((T, k)).astype(np.float32)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(y, torch.from_numpy(pos).to(DEV), torch.from_numpy(w).to(DEV), T, k, H, R,
                    out, ys, S)
    torch.cuda.synchronize()
    ref = orc.combine(bf(y), pos, w.astype(np.float64), bf(ys))
    assert_close(bf(out), ref, 2 ** -8, "combine")


def _ffn_case(E, R, H, I, offsets, seed, shared=False):
    wl = wk.WORKLOADS["mid_t2048"].scaled(seed=seed)
    xp = wk.normal_bf16(wl, "x", 20, (R, H), 1.0, DEV)
    w1 = wk.normal_bf16(wl, "w1", 20, (E, 2 * I, H), 0.02, DEV)
    w2 = wk.normal_bf16(wl, "w2", 20, (E, H, I), 0.02, DEV)
    return xp, w1, w2


@pytest.mark.parametrize("shape", [
    # E, H, I, offsets (ragged, an empty expert, one-row expert, tails in M and in I)
    (5, 512, 320, [0, 300, 300, 813, 999, 1000]),
    (3, 1024, 384, [0, 256, 512, 1025]),
    (1, 256, 512, [0, 7]),
    # K loops of one and two steps with 64-row tiles only (the deeper ring's empty steps)
    (3, 64, 64, [0, 10, 10, 70]),
    (2, 128, 128, [0, 33, 97]),
])
def test_expert_ffn_bf16_parity(shape):
    E, H, I, off = shape
    R = off[-1]
    xp, w1, w2 = _ffn_case(E, R, H, I, off, 1)
    offs = torch.tensor(off, dtype=torch.int32, device=DEV)
    y = torch.empty(R, H, dtype=torch.bfloat16, device=DEV)
    gu = torch.empty(R, 2 * I, dtype=torch.bfloat16, device=DEV)
    h = torch.empty(R, I, dtype=torch.bfloat16, device=DEV)
    moe.moe_expert_ffn(moe.BF16, xp, offs, E, R, H, I, w1, w2, y, gu_save=gu, h_save=h)
    torch.cuda.synchronize()
    ry, rgu, rh = orc.ffn_fwd(bf(xp), np.array(off, np.int32), bf(w1), bf(w2), want_gu=True,
                              want_h=True)
    assert_close(bf(gu), rgu, TOL_BF16, "gu")
    assert_close(bf(h), rh, TOL_BF16, "h")
    assert_close(bf(y), ry, TOL_BF16, "y")


def test_expert_ffn_shared_mode():
    E, R, H, I = 2, 300, 512, 256
    xp, w1, w2 = _ffn_case(E, R, H, I, None, 2)
    y = torch.empty(E, R, H, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.ffn_workspace_size(moe.BF16, E, R, H, I, True), dtype=torch.uint8,
                     device=DEV)
    moe.moe_expert_ffn(moe.BF16, xp, None, E, R, H, I, w1, w2, y, ws=ws)
    torch.cuda.synchronize()
    ry, _, _ = orc.ffn_fwd(bf(xp), None, bf(w1), bf(w2))
    assert_close(bf(y), ry, TOL_BF16, "y_shared")


@pytest.mark.parametrize("shape", [
    # E, H, I, offsets (None: shared experts, every expert on all R rows)
    (3, 512, 384, [0, 200, 201, 700]),
    (4, 256, 256, [0, 0, 300, 813, 1030]),  # an empty expert; several 256-row blocks
    (1, 128, 128, [0, 7]),                  # one-step K loops; one block of 7 rows
    (2, 384, 256, None),                    # shared mode, 300 rows per expert
], ids=["ragged", "empty_expert", "one_step_k", "shared"])
def test_expert_ffn_mxfp8_parity(shape):
    """The MXFP8 products (GEMM1's epilogue writes h's panel scales for GEMM2): y and the
    saves against the oracle, and a second call on a workspace holding other garbage
    bit-identical."""
    E, H, I, off = shape
    R = off[-1] if off else 300
    print(f"  case E={E} H={H} I={I} offsets={off}", flush=True)
    shared = off is None
    xp, w1, w2 = _ffn_case(E, R, H, I, off, 3)
    q = lambda rows, K: (torch.empty(rows, K, dtype=torch.uint8, device=DEV),
                         torch.empty(rows, K // 32, dtype=torch.uint8, device=DEV))
    xq, xs = q(R, H)
    w1q, w1s = q(E * 2 * I, H)
    w2q, w2s = q(E * H, I)
    moe.mx_quantize(xp, moe.BF16, R, H, xq, xs)
    moe.mx_quantize(w1, moe.BF16, E * 2 * I, H, w1q, w1s)
    moe.mx_quantize(w2, moe.BF16, E * H, I, w2q, w2s)
    offs = None if shared else torch.tensor(off, dtype=torch.int32, device=DEV)
    rows = E * R if shared else R
    outs = []
    for fill in (0xA5, 0xFF):  # garbage in the workspace: the call clears what it needs
        y = torch.full((rows, H), -1.0, dtype=torch.bfloat16, device=DEV)
        gu = torch.full((rows, 2 * I), -1.0, dtype=torch.bfloat16, device=DEV)
        h = torch.full((rows, I), -1.0, dtype=torch.bfloat16, device=DEV)
        ws = torch.full((moe.ffn_workspace_size(moe.MXFP8, E, R, H, I, shared),), fill,
                        dtype=torch.uint8, device=DEV)
        moe.moe_expert_ffn(moe.MXFP8, xq, offs, E, R, H, I, w1q, w2q, y, xp_scales=xs,
                           w1_scales=w1s, w2_scales=w2s, gu_save=gu, h_save=h, ws=ws)
        torch.cuda.synchronize()
        outs.append((y, gu, h))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    y, gu, h = outs[0]
    dq = lambda a: orc.mx_dequantize(*orc.mx_quantize(a))
    ry, rgu, rh = orc.ffn_fwd(dq(bf(xp)), None if shared else np.array(off, np.int32),
                              dq(bf(w1)), dq(bf(w2)), h_mx=True, want_gu=True, want_h=True)
    assert_close(bf(gu), rgu, TOL_BF16, "gu")
    assert_close(bf(h), rh, TOL_MX, "h")
    assert_close(bf(y).reshape(ry.shape), ry, TOL_MX, "y_mx")


def _ffn_forms(E, R, H, I, off, seed):
    """The BF16 FFN in its three forms: two launches without a workspace (h and g|u saved),
    one queue launch with a workspace and the g|u save, and one queue launch without the
    save.  Returns (y, gu, h, ws) of each."""
    xp, w1, w2 = _ffn_case(E, R, H, I, off, seed)
    offs = torch.tensor(off, dtype=torch.int32, device=DEV)
    outs = []
    for use_ws, save_gu in ((False, True), (True, True), (True, False)):
        y = torch.full((R, H), -1.0, dtype=torch.bfloat16, device=DEV)
        gu = torch.full((R, 2 * I), -1.0, dtype=torch.bfloat16, device=DEV) if save_gu else None
        h = torch.full((R, I), -1.0, dtype=torch.bfloat16, device=DEV)
        ws = None
        if use_ws:  # garbage in the workspace: the call clears what it needs
            ws = torch.full((moe.ffn_workspace_size(moe.BF16, E, R, H, I),), 0xA5,
                            dtype=torch.uint8, device=DEV)
        moe.moe_expert_ffn(moe.BF16, xp, offs, E, R, H, I, w1, w2, y, gu_save=gu, h_save=h,
                           ws=ws)
        torch.cuda.synchronize()
        outs.append((y, gu, h, ws))
    return outs


@pytest.mark.parametrize("shape", [
    (5, 512, 320, [0, 300, 300, 813, 999, 1000]),
    (3, 1024, 384, [0, 256, 512, 1025]),
    (1, 256, 512, [0, 7]),
    (4, 7168, 2048, [0, 1322, 9292, 13050, 16384]),  # the EP-64 share's realised loads
    (3, 64, 64, [0, 10, 10, 70]),                     # one-step K loops, 64-row tiles
], ids=["ragged", "tails", "one_expert_7_rows", "ep64_share", "one_step_k"])
def test_expert_ffn_one_launch_bit_identical(shape):
    """One launch of both products (tile queue with per-row-block dependencies) against the
    two launches: every output bit for bit, the error word zero."""
    E, H, I, off = shape
    R = off[-1]
    print(f"ffn one-launch case E={E} H={H} I={I} R={R}", flush=True)
    (y0, gu0, h0, _), (y1, gu1, h1, ws1), (y2, _, h2, ws) = _ffn_forms(E, R, H, I, off, 11)
    assert moe.ffn_error(ws) == 0 and moe.ffn_error(ws1) == 0
    assert torch.equal(gu0, gu1)
    for y, h in ((y1, h1), (y2, h2)):
        assert torch.equal(y0, y) and torch.equal(h0, h)


def test_expert_ffn_one_launch_parity_and_reuse():
    """The queue form against the oracle; then the same workspace serves a second, smaller
    call (its counters are cleared again)."""
    E, H, I = 4, 512, 256
    off = [0, 700, 700, 1100, 1500]
    xp, w1, w2 = _ffn_case(E, off[-1], H, I, off, 12)
    ws = torch.full((moe.ffn_workspace_size(moe.BF16, E, off[-1], H, I),), 0xFF,
                    dtype=torch.uint8, device=DEV)
    for offs in (off, [0, 100, 333, 333, 600]):
        R = offs[-1]
        y = torch.empty(R, H, dtype=torch.bfloat16, device=DEV)
        moe.moe_expert_ffn(moe.BF16, xp[:R], torch.tensor(offs, dtype=torch.int32, device=DEV),
                           E, R, H, I, w1, w2, y, ws=ws)
        torch.cuda.synchronize()
        assert moe.ffn_error(ws) == 0
        ry, _, _ = orc.ffn_fwd(bf(xp[:R]), np.array(offs, np.int32), bf(w1), bf(w2))
        assert_close(bf(y), ry, TOL_BF16, f"y_queue_R{R}")


@pytest.mark.parametrize("mode", [moe.MX_FLOOR, moe.MX_CEIL])
def test_mx_encoder_every_rounding_case(mode):
    """The E4M3 encoder on every rounding situation: each block holds 511 (block maximum:
    scale exponent 0 in floor mode, so the other values reach the encoder unscaled; 1 in ceil
    mode) and 31 fp32 values below 511 in magnitude whose upper 16 bits run over every sign,
    exponent and top-7 mantissa pattern, each with low 16 bits 0 (exact or a tie at the
    rounding bit), 1 (just above a tie), 0x7FFF, 0x8000, 0x8001 and 0xFFFF (sticky bits), so
    ties, near-ties, subnormal codes, flushes to zero and saturation at 448 all occur."""
    hi = np.arange(65536, dtype=np.uint32)
    exp = (hi >> 7) & 0xFF
    hi = hi[exp <= 135]  # |v| < 512
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    vals = ((hi[:, None] << 16) | lo[None, :]).ravel().view(np.float32)
    vals = vals[np.abs(vals) < 511.0]
    nb = -(-len(vals) // 31)
    blocks = np.zeros((nb, 32), np.float32)
    blocks[:, 0] = 511.0
    flat = np.zeros(nb * 31, np.float32)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(nb, 31)
    nb8 = -(-nb // 8) * 8
    blocks = np.concatenate([blocks, np.zeros((nb8 - nb, 32), np.float32)])
    f = blocks.reshape(-1, 256)
    rows = f.shape[0]
    q = torch.empty(rows, 256, dtype=torch.uint8, device=DEV)
    s = torch.empty(rows, 8, dtype=torch.uint8, device=DEV)
    moe.mx_quantize(torch.from_numpy(f).to(DEV), moe.F32, rows, 256, q, s, mode)
    torch.cuda.synchronize()
    rq, rsc = orc.mx_quantize(f.astype(np.float64), mode)
    assert np.array_equal(host(s), rsc)
    assert np.array_equal(host(q), rq)


def test_expert_ffn_one_launch_shared_mode_bit_identical():
    """Shared experts (offsets null: every expert takes all rows) through the one-launch
    queue against the two launches, bit for bit."""
    E, R, H, I = 3, 700, 512, 384
    xp, w1, w2 = _ffn_case(E, R, H, I, None, 13)
    outs = []
    for use_ws in (False, True):
        y = torch.full((E, R, H), -1.0, dtype=torch.bfloat16, device=DEV)
        h = torch.full((E, R, I), -1.0, dtype=torch.bfloat16, device=DEV)
        ws = None
        if use_ws:
            ws = torch.full((moe.ffn_workspace_size(moe.BF16, E, R, H, I, True),), 0x5A,
                            dtype=torch.uint8, device=DEV)
        moe.moe_expert_ffn(moe.BF16, xp, None, E, R, H, I, w1, w2, y, h_save=h, ws=ws)
        torch.cuda.synchronize()
        outs.append((y, h, ws))
    assert moe.ffn_error(outs[1][2]) == 0
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_route_selection_only_and_loads_only():
    """moe_route without permutation outputs (selection only) and with counts and offsets alone
    (the loads): the outputs it does write equal those of the full call, bit for bit."""
    T, E, k = 2048, 256, 8
    L = torch.from_numpy(np.random.default_rng(21).standard_normal((T, E)).astype(np.float32)).to(DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    ws = torch.empty(max(moe.route_workspace_size(T, k, E), 256), dtype=torch.uint8, device=DEV)
    outs = []
    for mode in ("full", "loads", "select"):
        o = dict(idx=torch.full((T, k), -7, **i32), w=torch.full((T, k), -7.0, device=DEV),
                 s_sel=torch.full((T, k), -7.0, device=DEV), counts=torch.full((E,), -7, **i32),
                 offsets=torch.full((E + 1,), -7, **i32), pos=torch.full((T, k), -7, **i32),
                 src=torch.full((T * k,), -7, **i32))
        kw = dict(o)
        if mode != "full":
            kw["pos"] = kw["src"] = None
        if mode == "select":
            kw["counts"] = kw["offsets"] = None
        moe.moe_route(L, T, E, k, score=wk.SIGMOID, ws=ws, **kw)
        torch.cuda.synchronize()
        outs.append(o)
    full, loads, select = outs
    for n in ("idx", "w", "s_sel"):
        assert torch.equal(loads[n], full[n]) and torch.equal(select[n], full[n]), n
    assert torch.equal(loads["counts"], full["counts"])
    assert torch.equal(loads["offsets"], full["offsets"])
    assert torch.all(loads["pos"] == -7) and torch.all(select["counts"] == -7)
