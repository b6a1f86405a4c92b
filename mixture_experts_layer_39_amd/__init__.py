"""Python binding of libmoe.so, the gfx950 deterministic mixture-of-experts layer library.

The functions here carry the names of the C ABI in ``include/moe.h`` and only marshal
arguments: tensors become device pointers, the current torch stream becomes the HIP stream,
and a negative return code becomes an exception.  Every step of the layer runs in the HIP
kernels of libmoe.so; there is no fallback of any kind.  torch supplies device memory and
streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EWORKSPACE, MOE_EHIP, MOE_EUNSUPPORTED = 0, -1, -2, -3, -4
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
BF16, MXFP8, F32 = 0, 1, 2
MX_FLOOR, MX_CEIL = 0, 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


class RouteCfg(ctypes.Structure):
    _fields_ = [("score", _i), ("n_groups", _i), ("topk_groups", _i), ("renorm", _i),
                ("route_scale", ctypes.c_float), ("sel_bias", _vp)]


class BwdArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("T", "H", "E", "k", "I", "R", "S", "Is", "E_router", "score",
                                  "renorm")] + [("route_scale", ctypes.c_float)] + \
               [(n, _vp) for n in ("x", "xp", "gu", "h", "y", "offsets", "pos", "idx", "w",
                                   "s_sel", "logits", "w1", "w2", "gus", "hs", "ws1", "ws2",
                                   "dout", "dx", "dw1", "dw2", "dws1", "dws2", "dw_route",
                                   "dlogits")] + \
               [(n, _i) for n in ("passes", "pass_tokens", "pass_rows", "mx")] + \
               [(n, _vp) for n in ("w2t_codes", "w2t_scales", "w1t_codes", "w1t_scales",
                                   "xp_codes", "xp_scales")]


class FwdArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("T", "H", "E", "k", "I", "S", "Is", "E_router")] + \
               [("cfg", RouteCfg)] + \
               [(n, _vp) for n in ("x", "w_router", "logits", "idx_in", "w1", "w2", "ws1", "ws2",
                                   "idx", "w", "s_sel", "counts", "offsets", "pos", "src", "xp",
                                   "gu", "h", "y", "gus", "hs", "ys", "out")]


_INT_FIELDS = ("T", "H", "E", "k", "I", "R", "S", "Is", "E_router", "score", "renorm", "passes",
               "pass_tokens", "pass_rows", "mx")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python mixture_experts_layer_39_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [_i]
        L.moe_abi_version.restype = _i
        L.moe_route_workspace_size.restype = _sz
        L.moe_route_workspace_size.argtypes = [_i, _i, _i]
        L.moe_route.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, ctypes.POINTER(RouteCfg), _vp,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_route_noalloc.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, ctypes.POINTER(RouteCfg),
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_dispatch.argtypes = [_vp, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp]
        L.moe_update_bias.argtypes = [_vp, _i, ctypes.c_float, _vp, _vp]
        L.moe_ffn_workspace_size.restype = _sz
        L.moe_ffn_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
        L.moe_ffn_error_offset.restype = _sz
        L.moe_ffn_error_offset.argtypes = []
        L.moe_expert_ffn.argtypes = [_i, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _sz, _vp]
        L.moe_combine.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _vp, _vp]
        L.moe_backward_workspace_size.restype = _sz
        L.moe_backward_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
        L.moe_backward.argtypes = [ctypes.POINTER(BwdArgs), _vp, _sz, _vp]
        L.moe_layer_forward_workspace_size.restype = _sz
        L.moe_layer_forward_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
        L.moe_layer_forward.argtypes = [ctypes.POINTER(FwdArgs), _vp, _sz, _vp]
        L.moe_layer_forward_error_offset.restype = _sz
        L.moe_layer_forward_error_offset.argtypes = [ctypes.POINTER(FwdArgs)]
        L.mx_quantize.argtypes = [_vp, _i, _i, _i, _vp, _vp, _i, _vp]
        L.mx_quantize_t.argtypes = [_vp, _i, _i, _i, _vp, _vp, _i, _vp]
        L.mx_dequantize.argtypes = [_vp, _vp, _i, _i, _vp, _vp]
        L.moe_trace_begin.argtypes = [_i]
        L.moe_trace_end.argtypes = []
        L.moe_trace_get.argtypes = [_i, ctypes.POINTER(ctypes.c_char_p),
                                    ctypes.POINTER(ctypes.c_float)]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def _p(t) -> _vp:
    if t is None:
        return None
    if isinstance(t, int):
        return _vp(t)
    return _vp(t.data_ptr())


def _stream(stream) -> _vp:
    if stream is None:
        if torch.cuda.is_available():
            return _vp(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return _vp(stream)
    return _vp(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


# ----------------------------------------------------------------------------- calls
def route_workspace_size(T: int, k: int, E: int) -> int:
    return lib().moe_route_workspace_size(T, k, E)


def moe_route(logits, T, E, k, *, x=None, w_router=None, H=0, score=SCORE_SOFTMAX,
              n_groups=1, topk_groups=1, renorm=True, route_scale=1.0, sel_bias=None,
              idx_in=None, idx=None, w=None, s_sel=None, counts, offsets, pos, src, ws,
              stream=None):
    cfg = RouteCfg(score, n_groups, topk_groups, int(renorm), route_scale,
                   None if sel_bias is None else sel_bias.data_ptr())
    rc = lib().moe_route(_p(logits), _p(x), _p(w_router), T, H, E, k, ctypes.byref(cfg),
                         _p(idx_in), _p(idx), _p(w), _p(s_sel), _p(counts), _p(offsets),
                         _p(pos), _p(src), _p(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                         _stream(stream))
    _check("moe_route", rc)


ROUTE_NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_route_noalloc(logits, T, E, k, *, x=None, w_router=None, H=0, score=SCORE_SOFTMAX,
                      n_groups=1, topk_groups=1, renorm=True, route_scale=1.0, sel_bias=None,
                      idx_in=None, idx=None, w=None, s_sel=None, counts, offsets, pos, src,
                      stream=None):
    """moe_route without a workspace: the library's static device scratch (callers that
    cannot allocate; calls that overlap on one device race)."""
    cfg = RouteCfg(score, n_groups, topk_groups, int(renorm), route_scale,
                   None if sel_bias is None else sel_bias.data_ptr())
    rc = lib().moe_route_noalloc(_p(logits), _p(x), _p(w_router), T, H, E, k, ctypes.byref(cfg),
                                 _p(idx_in), _p(idx), _p(w), _p(s_sel), _p(counts), _p(offsets),
                                 _p(pos), _p(src), _stream(stream))
    _check("moe_route_noalloc", rc)


def moe_update_bias(counts, E, gamma, bias, stream=None):
    rc = lib().moe_update_bias(_p(counts), E, float(gamma), _p(bias), _stream(stream))
    _check("moe_update_bias", rc)


def moe_dispatch(x, T, H, k, src, R, xp=None, xp_codes=None, xp_scales=None, stream=None,
                 pos=None):
    rc = lib().moe_dispatch(_p(x), T, H, k, _p(src), _p(pos), R, _p(xp), _p(xp_codes),
                            _p(xp_scales), _stream(stream))
    _check("moe_dispatch", rc)


def ffn_workspace_size(dtype, E, R, H, I, shared=False) -> int:
    return lib().moe_ffn_workspace_size(dtype, E, R, H, I, int(shared))


def ffn_error(ws) -> int:
    """The one-launch FFN's error word in `ws` (0: every wait completed).  Reads the device."""
    off = lib().moe_ffn_error_offset()
    return int(ws[off:off + 4].view(torch.int32).item())


def moe_expert_ffn(dtype, xp, offsets, E, R, H, I, w1, w2, y, *, xp_scales=None,
                   w1_scales=None, w2_scales=None, gu_save=None, h_save=None, ws=None,
                   stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    rc = lib().moe_expert_ffn(dtype, _p(xp), _p(xp_scales), _p(offsets), E, R, H, I, _p(w1),
                              _p(w1_scales), _p(w2), _p(w2_scales), _p(gu_save), _p(h_save),
                              _p(y), _p(ws), nbytes, _stream(stream))
    _check("moe_expert_ffn", rc)


def moe_combine(y, pos, w, T, k, H, R, out, ys=None, S=0, stream=None):
    rc = lib().moe_combine(_p(y), _p(pos), _p(w), T, k, H, R, _p(ys), S, _p(out),
                           _stream(stream))
    _check("moe_combine", rc)


def bwd_args(**kw) -> BwdArgs:
    a = BwdArgs()
    for name, _ in BwdArgs._fields_:
        v = kw.get(name)
        if v is None:
            continue
        if name == "route_scale":
            a.route_scale = float(v)
        elif isinstance(v, (bool, int)) and name in _INT_FIELDS:
            setattr(a, name, int(v))
        else:
            setattr(a, name, v if isinstance(v, int) else v.data_ptr())
    return a


def backward_workspace_size(a: BwdArgs) -> int:
    return lib().moe_backward_workspace_size(ctypes.byref(a))


def moe_backward(a: BwdArgs, ws, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    rc = lib().moe_backward(ctypes.byref(a), _p(ws), nbytes, _stream(stream))
    _check("moe_backward", rc)


def mx_quantize_t(inp, batch, A, B, codes, scales, scale_mode=MX_FLOOR, stream=None):
    rc = lib().mx_quantize_t(_p(inp), batch, A, B, _p(codes), _p(scales), scale_mode,
                             _stream(stream))
    _check("mx_quantize_t", rc)


def mx_dequantize(codes, scales, rows, K, out, stream=None):
    rc = lib().mx_dequantize(_p(codes), _p(scales), rows, K, _p(out), _stream(stream))
    _check("mx_dequantize", rc)


def fwd_args(*, score=SCORE_SOFTMAX, n_groups=1, topk_groups=1, renorm=True, route_scale=1.0,
             sel_bias=None, **kw) -> FwdArgs:
    """Arguments of moe_layer_forward: sizes as ints, tensors (or raw device addresses)."""
    a = FwdArgs()
    a.cfg = RouteCfg(score, n_groups, topk_groups, int(renorm), route_scale,
                     None if sel_bias is None else sel_bias.data_ptr())
    for name, _ in FwdArgs._fields_:
        v = kw.get(name)
        if name == "cfg" or v is None:
            continue
        if name in ("T", "H", "E", "k", "I", "S", "Is", "E_router"):
            setattr(a, name, int(v))
        else:
            setattr(a, name, v if isinstance(v, int) else v.data_ptr())
    return a


def layer_forward_workspace_size(a: FwdArgs) -> int:
    return lib().moe_layer_forward_workspace_size(ctypes.byref(a))


def layer_forward_error(a: FwdArgs, ws) -> int:
    """The single launch's error word in `ws` (0: every wait completed).  Reads the device."""
    off = lib().moe_layer_forward_error_offset(ctypes.byref(a))
    return int(ws[off:off + 4].view(torch.int32).item())


def moe_layer_forward(a: FwdArgs, ws, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    rc = lib().moe_layer_forward(ctypes.byref(a), _p(ws), nbytes, _stream(stream))
    _check("moe_layer_forward", rc)


def mx_quantize(inp, in_dtype, rows, K, codes, scales, scale_mode=MX_FLOOR, stream=None):
    rc = lib().mx_quantize(_p(inp), in_dtype, rows, K, _p(codes), _p(scales), scale_mode,
                           _stream(stream))
    _check("mx_quantize", rc)


# ----------------------------------------------------------------------------- tracing
def trace_begin(cap: int = 4096):
    """Arm per-launch event tracing of the library's kernels on this thread."""
    _check("moe_trace_begin", lib().moe_trace_begin(cap))


def trace_end() -> list[tuple[str, float]]:
    """Disarm tracing; returns (role name, milliseconds) of every recorded launch, in order
    (waits for the launches to finish)."""
    L = lib()
    n = L.moe_trace_end()
    out = []
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    for i in range(n):
        _check("moe_trace_get", L.moe_trace_get(i, ctypes.byref(name), ctypes.byref(ms)))
        out.append((name.value.decode(), float(ms.value)))
    return out
