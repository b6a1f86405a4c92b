"""CPU oracle of the deterministic mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library (``mixture_experts_layer_39_amd``) never imports
it, and the two share no code: the only common module is ``workloads`` (seeded inputs).

``moe_oracle.c`` holds the arithmetic (fp64, plain loops; see its header).  This module
builds it with gcc, binds it with ctypes, and composes its steps into the whole layer.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; the process must preload libasan), used by the sanitizer pin run.
SANITIZE = os.environ.get("MOE_ORACLE_SANITIZE", "") == "1"
_LIB = os.path.join(_HERE, "libmoe_oracle_san.so" if SANITIZE else "libmoe_oracle.so")
_lib = None

SOFTMAX, SIGMOID = 0, 1

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool | None = None) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction); with
    `sanitize`, the AddressSanitizer + UndefinedBehaviorSanitizer build."""
    san = SANITIZE if sanitize is None else sanitize
    out = os.path.join(_HERE, "libmoe_oracle_san.so" if san else "libmoe_oracle.so")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared"] + (SAN_FLAGS if san else [])
                              + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_rsig.restype = ctypes.c_float
        _lib.orc_rsig.argtypes = [ctypes.c_float]
        _lib.orc_e4m3_decode.restype = ctypes.c_double
        _lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.orc_e4m3_encode.restype = ctypes.c_uint8
        _lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- steps
def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_to_f64(_p(b), ctypes.c_int64(b.size), _p(out))
    return out


def router_logits(x_bf16: np.ndarray, wr_bf16: np.ndarray) -> np.ndarray:
    x, wr = _c(x_bf16, np.uint16), _c(wr_bf16, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(_p(x), _p(wr), T, H, E, _p(out))
    return out


def rsig(x: float) -> np.float32:
    return np.float32(lib().orc_rsig(float(x)))


def route_select(logits, k, score=SOFTMAX, n_groups=1, topk_groups=1, bias=None):
    L = _c(logits, np.float32)
    T, E = L.shape
    idx = np.empty((T, k), np.int32)
    s_sel = np.empty((T, k), np.float32)
    b = None if bias is None else _c(bias, np.float32)
    rc = lib().orc_route_select(_p(L), T, E, k, score, n_groups, topk_groups, _p(b),
                                _p(idx), _p(s_sel))
    if rc != 0:
        raise ValueError("invalid routing configuration")
    return idx, s_sel


def route_weights(logits, idx, score=SOFTMAX, renorm=True, route_scale=1.0):
    L = _c(logits, np.float64)
    idx = _c(idx, np.int32)
    T, E = L.shape
    k = idx.shape[1]
    w = np.empty((T, k), np.float64)
    lib().orc_route_weights(_p(L), _p(idx), T, E, k, score, int(renorm),
                            ctypes.c_double(route_scale), _p(w))
    return w


def permute(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pos = np.empty((T, k), np.int32)
    src = np.empty(T * k, np.int32)
    lib().orc_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(pos), _p(src))
    return counts, offsets, pos, src


def update_bias(counts, bias, gamma):
    """Load-balancing bias update (auxiliary-loss-free balancing of DeepSeek-V3): returns the
    new fp32 bias; see ``orc_update_bias``."""
    c = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    lib().orc_update_bias(_p(c), int(c.size), ctypes.c_float(gamma), _p(b))
    return b


def dispatch(x_bf16, k, src):
    x = _c(x_bf16, np.uint16)
    src = _c(src, np.int32)
    T, H = x.shape
    xp = np.empty((len(src), H), np.uint16)
    lib().orc_dispatch(_p(x), T, H, k, _p(src), len(src), _p(xp))
    return xp


def ffn_fwd(xp, offsets, w1, w2, h_mx=False, want_gu=False, want_h=False):
    """xp [R,H] f64; offsets [E+1] or None (every expert takes all rows); w1 [E,2I,H],
    w2 [E,H,I] f64.  Returns y ([R,H], or [E,R,H] when offsets is None), gu, h."""
    xp, w1, w2 = _c(xp, np.float64), _c(w1, np.float64), _c(w2, np.float64)
    R, H = xp.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    off = None if offsets is None else _c(offsets, np.int32)
    rows = R if off is not None else E * R
    y = np.empty((rows, H), np.float64)
    gu = np.empty((rows, 2 * I), np.float64) if want_gu else None
    h = np.empty((rows, I), np.float64) if want_h else None
    lib().orc_ffn_fwd(_p(xp), _p(off), E, R, H, I, _p(w1), _p(w2), int(h_mx), _p(gu),
                      _p(h), _p(y))
    if off is None:
        y = y.reshape(E, R, H)
    return y, gu, h


def combine(y, pos, w, ys=None):
    y, pos, w = _c(y, np.float64), _c(pos, np.int32), _c(w, np.float64)
    T, k = pos.shape
    H = y.shape[1]
    S = 0 if ys is None else ys.shape[0]
    ys_ = None if ys is None else _c(ys, np.float64)
    out = np.empty((T, H), np.float64)
    lib().orc_combine(_p(y), _p(pos), _p(w), T, k, H, _p(ys_), S, _p(out))
    return out


def combine_bwd(dout, y, pos, w):
    dout, y, pos, w = (_c(dout, np.float64), _c(y, np.float64), _c(pos, np.int32),
                       _c(w, np.float64))
    T, k = pos.shape
    H = y.shape[1]
    dy = np.zeros_like(y)
    dw = np.empty((T, k), np.float64)
    lib().orc_combine_bwd(_p(dout), _p(y), _p(pos), _p(w), T, k, H, _p(dy), _p(dw))
    return dy, dw


def ffn_bwd(xp, offsets, w1, w2, dy):
    xp, w1, w2, dy = (_c(xp, np.float64), _c(w1, np.float64), _c(w2, np.float64),
                      _c(dy, np.float64))
    R, H = xp.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    off = None if offsets is None else _c(offsets, np.int32)
    rows = R if off is not None else E * R
    dxp = np.empty((rows, H), np.float64)
    dw1 = np.empty_like(w1)
    dw2 = np.empty_like(w2)
    lib().orc_ffn_bwd(_p(xp), _p(off), E, R, H, I, _p(w1), _p(w2), _p(dy), _p(dxp),
                      _p(dw1), _p(dw2))
    if off is None:
        dxp = dxp.reshape(E, R, H)
    return dxp, dw1, dw2


def bf16_round(a):
    """Values rounded to bf16 (through fp32, to nearest even), as f64."""
    b = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32)).view(np.uint32)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32).astype(np.float64)


def mx_tokens(x):
    """x [M, C] f64 MX-quantised along its first (token) dimension, in 32-row blocks from row 0
    (a partial last block padded with zeros), returned dequantised, [M, C]."""
    x = _c(x, np.float64)
    M, C = x.shape
    Mp = -(-M // 32) * 32
    xt = np.zeros((C, Mp))
    xt[:, :M] = x.T
    return mx_dequantize(*mx_quantize(xt))[:, :M].T


def ffn_bwd_mx(xp, offsets, w1, w2, dy, gu, h, mx_wgrad=False):
    """Backward of the routed FFN after an MXFP8 forward, with MXFP8 dgrad products.

    The two dgrad products take MX-quantised operands along their contraction dimension
    (E4M3 codes, one E8M0 scale per 32 values, the MOE_MX_FLOOR rule of mx_quantize):
      dh   = Q_H(dy) . Q_H(W2_e)^T      (dy per row along H; W2_e [H,I] per column, along H)
      dGU  = SwiGLU backward of dh at the saved g|u   (fp64)
      dXp  = Q_2I(dGU) . Q_2I(W1_e)^T   (dGU per row along 2I; W1_e [2I,H] per column)
    The weight gradients are sums over the expert's rows of dy and dGU against the forward's
    GEMM inputs (h and xp as the forward consumed them):
      dW2_e = dy_e^T h_e,   dW1_e = dGU_e^T xp_e,
    in fp64 from the unquantised values, or with mx_wgrad every operand MX-quantised along the
    expert's tokens (32-row blocks from the expert's first row, mx_tokens).
    dy and dGU are quantised from their bf16 values (bf16_round): the precision the kernels
    hold them in when they take the quantisation decisions.
    xp [R,H], dy [R,H], gu [R,2I], h [R,I] f64; w1 [E,2I,H], w2 [E,H,I] f64 (bf16 values).
    Returns dxp [R,H], dgu [R,2I], dw1, dw2.
    """
    xp, dy, gu, h = (_c(xp, np.float64), _c(dy, np.float64), _c(gu, np.float64),
                     _c(h, np.float64))
    w1, w2 = _c(w1, np.float64), _c(w2, np.float64)
    off = _c(offsets, np.int32)
    E, I2, H = w1.shape
    I = I2 // 2
    R = xp.shape[0]
    dyb = bf16_round(dy)
    dyq = mx_dequantize(*mx_quantize(dyb)) if R else dy
    dxp = np.zeros((R, H))
    dgu = np.zeros((R, 2 * I))
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        w2t = mx_dequantize(*mx_quantize(np.ascontiguousarray(w2[e].T)))   # [I,H], along H
        w1t = mx_dequantize(*mx_quantize(np.ascontiguousarray(w1[e].T)))   # [H,2I], along 2I
        dh = dyq[r0:r1] @ w2t.T
        g, u = gu[r0:r1, :I], gu[r0:r1, I:]
        sg = 1.0 / (1.0 + np.exp(-g))
        dgu[r0:r1, :I] = dh * u * sg * (1.0 + g * (1.0 - sg))
        dgu[r0:r1, I:] = dh * g * sg
        dgub = bf16_round(dgu[r0:r1])
        dguq = mx_dequantize(*mx_quantize(dgub))
        dxp[r0:r1] = dguq @ w1t.T
        if mx_wgrad:
            dw2[e] = mx_tokens(dyb[r0:r1]).T @ mx_tokens(h[r0:r1])
            dw1[e] = mx_tokens(dgub).T @ mx_tokens(xp[r0:r1])
        else:
            dw2[e] = dy[r0:r1].T @ h[r0:r1]
            dw1[e] = dgu[r0:r1].T @ xp[r0:r1]
    return dxp, dgu, dw1, dw2


def unpermute(dxp, pos, dxs=None):
    dxp, pos = _c(dxp, np.float64), _c(pos, np.int32)
    T, k = pos.shape
    H = dxp.shape[1]
    S = 0 if dxs is None else dxs.shape[0]
    dxs_ = None if dxs is None else _c(dxs, np.float64)
    dx = np.empty((T, H), np.float64)
    lib().orc_unpermute(_p(dxp), _p(pos), T, k, H, _p(dxs_), S, _p(dx))
    return dx


def router_bwd(logits, idx, dw, score=SOFTMAX, renorm=True, route_scale=1.0):
    L, idx, dw = _c(logits, np.float64), _c(idx, np.int32), _c(dw, np.float64)
    T, E = L.shape
    k = idx.shape[1]
    dL = np.empty((T, E), np.float64)
    lib().orc_router_bwd(_p(L), _p(idx), _p(dw), T, E, k, score, int(renorm),
                         ctypes.c_double(route_scale), _p(dL))
    return dL


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def mx_quantize(a, mode=0):
    a = _c(a, np.float64)
    K = a.shape[-1]
    rows = a.size // K
    codes = np.empty(a.shape, np.uint8)
    scales = np.empty(a.shape[:-1] + (K // 32,), np.uint8)
    lib().orc_mx_quantize(_p(a), ctypes.c_int64(rows), K, mode, _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes, scales):
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    K = codes.shape[-1]
    out = np.empty(codes.shape, np.float64)
    lib().orc_mx_dequantize(_p(codes), _p(scales), ctypes.c_int64(codes.size // K), K,
                            _p(out))
    return out


# ----------------------------------------------------------------------------- the layer
def _vals(a) -> np.ndarray:
    """A layer input as fp64 values: bf16 bit patterns (uint16) are converted exactly; fp64
    arrays are taken as they are (the finite-difference pins perturb them continuously)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    if a.dtype != np.float64:
        raise TypeError("layer inputs are bf16 bit patterns (uint16) or fp64 values")
    return np.ascontiguousarray(a)


def _gather_rows(x, k, src) -> np.ndarray:
    """Dispatch of [T,H] rows by src: bf16 bits through orc_dispatch, fp64 values through the
    same byte copy (each fp64 value is four 16-bit words of its row)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return dispatch(x, k, src)
    x = np.ascontiguousarray(x, np.float64)
    T, H = x.shape
    words = dispatch(x.view(np.uint16).reshape(T, 4 * H), k, src)
    return words.view(np.float64).reshape(len(src), H)


def layer_forward(p: dict) -> dict:
    """Whole forward of the layer.

    p: x [T,H]; logits [T,ER] (or w_router [ER,H] bf16 bits); k; score; renorm; route_scale;
    n_groups; topk_groups; bias (optional); w1/w2 [E,..]; optional idx_local [T,k'] (one
    GPU's share: local expert per routed pair) with E; optional ws1/ws2 (shared experts);
    mx (bool).  x and the weights are bf16 bit patterns (uint16), or fp64 values (BF16 path
    only).  The logits select in fp32 (as given in fp32, or rounded from fp64 values) and
    weight in fp64.
    Returns every intermediate the backward needs plus `out` [T,H] f64.
    """
    r = {}
    if "w_router" in p:
        r["logits"] = router_logits(p["x"], p["w_router"])
    elif np.asarray(p["logits"]).dtype == np.float64:
        r["logits"] = np.ascontiguousarray(p["logits"])
    else:
        r["logits"] = _c(p["logits"], np.float32)
    idx, s_sel = route_select(r["logits"].astype(np.float32), p["k"], p["score"],
                              p.get("n_groups", 1), p.get("topk_groups", 1), p.get("bias"))
    r["idx"], r["s_sel"] = idx, s_sel
    r["w"] = route_weights(r["logits"].astype(np.float64), idx, p["score"],
                           p.get("renorm", True), p.get("route_scale", 1.0))
    E = p["w1"].shape[0]
    lidx = p.get("idx_local", idx)
    kk = lidx.shape[1]
    counts, offsets, pos, src = permute(lidx, E)
    r.update(counts=counts, offsets=offsets, pos=pos, src=src)
    xp_rows = _gather_rows(p["x"], kk, src)
    if xp_rows.dtype == np.uint16:
        r["xp_bits"] = xp_rows
    w1 = _vals(p["w1"])
    w2 = _vals(p["w2"])
    xp = _vals(xp_rows)
    mx = p.get("mx", False)
    if mx:
        if np.asarray(p["x"]).dtype != np.uint16:
            raise TypeError("the MXFP8 forward takes bf16 inputs")
        xq = mx_quantize(xp)
        xp = mx_dequantize(*xq)
        w1 = mx_dequantize(*mx_quantize(w1))
        w2 = mx_dequantize(*mx_quantize(w2))
    r["xp"] = xp
    y, gu, h = ffn_fwd(xp, offsets, w1, w2, h_mx=mx, want_gu=True, want_h=True)
    r.update(y=y, gu=gu, h=h)
    ys = None
    x64 = _vals(p["x"])
    r["x"] = x64
    if p.get("ws1") is not None and p["ws1"].shape[0] > 0:
        ws1, ws2 = _vals(p["ws1"]), _vals(p["ws2"])
        ys, _, _ = ffn_fwd(x64, None, ws1, ws2)
        r["ys"] = ys
    r["out"] = combine(y, pos, r["w"], ys)
    return r


def layer_backward(p: dict, r: dict, dout) -> dict:
    """Whole backward in fp64 given the forward record `r`: BF16-storage products, or after
    an MXFP8 forward (p["mx"]) MXFP8 dgrad products, and with p["mx_wgrad"] MXFP8 weight-
    gradient products too (ffn_bwd_mx).  dout [T,H]: bf16 bits or fp64 values.
    Returns dx, dw1, dw2 (and dws1, dws2 with shared experts), dw_route [T,k] and dlogits."""
    dout = _vals(dout)
    w1, w2 = _vals(p["w1"]), _vals(p["w2"])
    dy, dw = combine_bwd(dout, r["y"], r["pos"], r["w"])
    if p.get("mx", False):
        dxp, _, dw1, dw2 = ffn_bwd_mx(r["xp"], r["offsets"], w1, w2, dy, r["gu"], r["h"],
                                      mx_wgrad=p.get("mx_wgrad", False))
    else:
        dxp, dw1, dw2 = ffn_bwd(r["xp"], r["offsets"], w1, w2, dy)
    g = {"dw_route": dw, "dw1": dw1, "dw2": dw2}
    dxs = None
    if p.get("ws1") is not None and p["ws1"].shape[0] > 0:
        ws1, ws2 = _vals(p["ws1"]), _vals(p["ws2"])
        S = ws1.shape[0]
        dys = np.broadcast_to(dout, (S,) + dout.shape).reshape(S * dout.shape[0], -1)
        dxs, dws1, dws2 = ffn_bwd(r["x"], None, ws1, ws2, dys)
        g["dws1"], g["dws2"] = dws1, dws2
    g["dx"] = unpermute(dxp, r["pos"], dxs)
    g["dlogits"] = router_bwd(r["logits"].astype(np.float64), r["idx"], dw, p["score"],
                              p.get("renorm", True), p.get("route_scale", 1.0))
    return g
