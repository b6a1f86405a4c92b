"""A whole MoE layer step as a sequence of the library's C-ABI calls.

``MoELayer`` owns the device buffers of one layer configuration (allocated once, with torch)
and runs forward (route -> dispatch -> expert FFN -> combine) and backward through
libmoe.so.  It holds no arithmetic: every value is produced by the HIP kernels.

Macrobatch ring (``ring_depth = D``; the ring buffer walked at minibatch granularity that the
pages describe, aiexpert.news "Megakernels are dead and back", ¶4): the tokens stream in
minibatches; each minibatch is routed on its own, and every D minibatches form a pass whose
routed rows are permuted into D ring slots, run through one grouped-GEMM pass and combined
back one minibatch at a time.  No token is dropped: every routed row of every minibatch is
dispatched, computed and combined exactly once.  Forward-only layers reuse one ring region
of D slots for every pass; training layers keep each pass's region for the backward, which
walks the passes again (one moe_backward call) and reduces the weight gradients over the
rows of every pass.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (BF16, MXFP8, F32, SCORE_SIGMOID, backward_workspace_size, bwd_args,
               ffn_workspace_size, fwd_args, layer_forward_workspace_size, moe_backward,
               moe_combine, moe_dispatch, moe_expert_ffn, moe_layer_forward, moe_route,
               moe_update_bias, mx_dequantize, mx_quantize, mx_quantize_t,
               route_workspace_size)


@dataclasses.dataclass
class LayerCfg:
    T: int
    H: int
    E: int
    k: int
    I: int
    S: int = 0
    Is: int = 0
    score: int = 0
    renorm: bool = True
    route_scale: float = 1.0
    n_groups: int = 1
    topk_groups: int = 1
    E_router: int = 0          # width of the router (0: E)
    local_share: bool = False  # expert of each routed pair comes from idx_local
    router_proj: bool = False
    mx: bool = False
    bias_gamma: float = 0.0    # > 0: sigmoid selection bias, updated from the loads each step
    mx_bwd: int = 2            # after an MXFP8 forward: 1 MXFP8 dgrad, BF16 weight gradients;
                               # 2 MXFP8 dgrad and weight gradients

    @property
    def ER(self):
        return self.E_router or self.E

    @staticmethod
    def from_workload(wl) -> "LayerCfg":
        return LayerCfg(T=wl.T, H=wl.H, E=wl.E, k=wl.k,
                        I=wl.I, S=wl.S, Is=wl.Is, score=wl.score, renorm=wl.renorm,
                        route_scale=wl.route_scale, n_groups=wl.n_groups,
                        topk_groups=wl.topk_groups, E_router=wl.E_router,
                        local_share=wl.local_share, router_proj=wl.router_proj, mx=wl.mx)


def _e(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


class MoELayer:
    def __init__(self, cfg: LayerCfg, inp: dict, device="cuda", backward: bool = True,
                 minibatch: int = 0, ring_depth: int = 0):
        c = self.cfg = cfg
        d = self.dev = torch.device(device)
        self.inp = inp
        T, H, E, I = c.T, c.H, c.E, c.I
        kr = inp["idx_local"].shape[1] if c.local_share else c.k  # routed slots per token
        if kr != c.k:
            raise ValueError("local share must have k routed rows per token")
        self.k_router = c.k
        self.kr = kr
        if c.bias_gamma > 0 and (c.score != SCORE_SIGMOID or minibatch):
            raise ValueError("the load-balancing bias applies to the sigmoid router of the "
                             "unstreamed layer")
        self.sel_bias = (torch.zeros(c.ER, dtype=torch.float32, device=d)
                         if c.bias_gamma > 0 else None)
        # macrobatch ring: minibatches of `minibatch` tokens, D of them per pass
        self.ring = minibatch > 0 and ring_depth > 0
        if self.ring:
            if c.local_share or c.mx or c.router_proj or c.S > 1:
                raise ValueError("ring mode supports routed layers with at most one shared expert")
            self.mb = minibatch
            self.n_mb = -(-T // minibatch)
            self.D = min(ring_depth, self.n_mb)
            self.passes = -(-self.n_mb // self.D)
            self.pass_tokens = self.D * minibatch
            self.pass_rows = self.pass_tokens * kr
            regions = self.passes if backward else 1
            R = self.R = regions * self.pass_rows
        else:
            R = self.R = T * kr
        ER = c.ER
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        # routing
        self.logits = inp["logits"] if "logits" in inp else _e((T, ER), f32, d)
        self.idx = _e((T, self.k_router), i32, d)
        self.w = _e((T, self.k_router), f32, d)
        self.s_sel = _e((T, self.k_router), f32, d)
        if self.ring:
            P = self.passes
            self.counts = _e((P, E), i32, d)
            self.offsets = _e((P, E + 1), i32, d)
            self.src = _e((P, self.pass_rows), i32, d)
        else:
            self.counts = _e((E,), i32, d)
            self.offsets = _e((E + 1,), i32, d)
            self.src = _e((R,), i32, d)
        self.pos = _e((T, kr), i32, d)
        self.route_ws = _e((max(route_workspace_size(T, kr, E),
                                route_workspace_size(T, self.k_router, ER), 256),),
                           torch.uint8, d)
        if c.local_share:   # the loads over the E_router experts (load-balancing bias)
            self.g_counts = _e((ER,), i32, d)
            self.g_offsets = _e((ER + 1,), i32, d)
        # expert FFN
        if c.mx:
            self.xq = _e((R, H), torch.uint8, d)
            self.xs = _e((R, H // 32), torch.uint8, d)
            self.w1q = _e(tuple(inp["w1"].shape), torch.uint8, d)
            self.w1s = _e(tuple(inp["w1"].shape[:-1]) + (H // 32,), torch.uint8, d)
            self.w2q = _e(tuple(inp["w2"].shape), torch.uint8, d)
            self.w2s = _e(tuple(inp["w2"].shape[:-1]) + (I // 32,), torch.uint8, d)
            if backward:
                # MXFP8 dgrad: the weights quantised along the dgrad contraction dimension;
                # the saves hold what the forward's GEMMs consumed
                self.w2tq = _e((E, I, H), torch.uint8, d)
                self.w2ts = _e((E, I, H // 32), torch.uint8, d)
                self.w1tq = _e((E, H, 2 * I), torch.uint8, d)
                self.w1ts = _e((E, H, 2 * I // 32), torch.uint8, d)
                # MXFP8 weight gradients read xp as the dispatch's codes; BF16 ones (mode 1)
                # need it dequantised
                self.xp = _e((R, H), bf, d) if c.mx_bwd != 2 else None
                self.gu = _e((R, 2 * I), bf, d)
                self.h = _e((R, I), bf, d)
            else:
                self.xp = None
                self.gu = self.h = None
            self.quantize_weights(backward)
        else:
            self.xp = _e((R, H), bf, d)
            self.gu = _e((R, 2 * I), bf, d) if backward else None
            self.h = _e((R, I), bf, d)
        self.y = _e((R, H), bf, d)
        self.ffn_ws = _e((max(ffn_workspace_size(MXFP8 if c.mx else BF16, E, R, H, I), 256),),
                         torch.uint8, d)
        if c.S:
            self.ys = _e((c.S, T, H), bf, d)
            self.gus = _e((c.S, T, 2 * c.Is), bf, d) if backward else None
            self.hs = _e((c.S, T, c.Is), bf, d)
            self.sh_ws = _e((max(ffn_workspace_size(BF16, c.S, T, H, c.Is, True), 256),),
                            torch.uint8, d)
        else:
            self.ys = None
        self.out = _e((T, H), bf, d)
        self.has_bwd = backward
        if backward:
            self.dx = _e((T, H), bf, d)
            self.dw1 = torch.empty_like(inp["w1"])
            self.dw2 = torch.empty_like(inp["w2"])
            self.dws1 = torch.empty_like(inp["ws1"]) if c.S else None
            self.dws2 = torch.empty_like(inp["ws2"]) if c.S else None
            self.dw_route = _e((T, kr), f32, d)
            self.dlogits = _e((T, ER), f32, d)
            self.bargs = self._bwd_args()
            self.bwd_ws = _e((max(backward_workspace_size(self.bargs), 256),), torch.uint8, d)

    # ------------------------------------------------------------------ setup
    def quantize_weights(self, backward=False):
        c, inp = self.cfg, self.inp
        E, H, I = c.E, c.H, c.I
        mx_quantize(inp["w1"], BF16, E * 2 * I, H, self.w1q, self.w1s)
        mx_quantize(inp["w2"], BF16, E * H, I, self.w2q, self.w2s)
        if backward:
            mx_quantize_t(inp["w2"], E, H, I, self.w2tq, self.w2ts)
            mx_quantize_t(inp["w1"], E, 2 * I, H, self.w1tq, self.w1ts)

    def _bwd_args(self):
        c, inp = self.cfg, self.inp
        ring = dict(passes=self.passes, pass_tokens=self.pass_tokens,
                    pass_rows=self.pass_rows) if self.ring else {}
        return bwd_args(**ring, T=c.T, H=c.H, E=c.E, k=self.kr, I=c.I, R=self.R, S=c.S, Is=c.Is,
                        E_router=c.ER, score=c.score, renorm=c.renorm,
                        route_scale=c.route_scale, x=inp["x"], xp=self.xp, gu=self.gu,
                        h=self.h, y=self.y, offsets=self.offsets, pos=self.pos, idx=self.idx,
                        w=self.w, s_sel=self.s_sel, logits=self.logits, w1=inp["w1"],
                        w2=inp["w2"], gus=self.gus if c.S else None,
                        hs=self.hs if c.S else None, ws1=inp.get("ws1"), ws2=inp.get("ws2"),
                        dout=inp.get("dout"), dx=self.dx, dw1=self.dw1, dw2=self.dw2,
                        dws1=self.dws1, dws2=self.dws2, dw_route=self.dw_route,
                        dlogits=self.dlogits,
                        **(dict(mx=c.mx_bwd, w2t_codes=self.w2tq, w2t_scales=self.w2ts,
                                w1t_codes=self.w1tq, w1t_scales=self.w1ts,
                                xp_codes=self.xq if c.mx_bwd == 2 else None,
                                xp_scales=self.xs if c.mx_bwd == 2 else None)
                           if c.mx else {}))

    # ------------------------------------------------------------------ steps
    def route(self):
        c, inp = self.cfg, self.inp
        common = dict(score=c.score, n_groups=c.n_groups, topk_groups=c.topk_groups,
                      renorm=c.renorm, route_scale=c.route_scale, ws=self.route_ws)
        if c.local_share:
            # the selection over all E_router experts (a permutation of it would feed the
            # exchange between GPUs, which one GPU's share does not have); the loads only
            # when the load-balancing bias needs them
            want_loads = c.bias_gamma > 0
            moe_route(self.logits, c.T, c.ER, self.k_router, idx=self.idx, w=self.w,
                      s_sel=self.s_sel, counts=self.g_counts if want_loads else None,
                      offsets=self.g_offsets if want_loads else None, pos=None, src=None,
                      sel_bias=self.sel_bias, **common)
            moe_route(None, c.T, c.E, self.kr, idx_in=inp["idx_local"], counts=self.counts,
                      offsets=self.offsets, pos=self.pos, src=self.src, **common)
            loads = self.g_counts
        else:
            moe_route(self.logits, c.T, c.E, c.k, x=inp["x"] if c.router_proj else None,
                      w_router=inp.get("w_router"), H=c.H, idx=self.idx, w=self.w,
                      s_sel=self.s_sel, counts=self.counts, offsets=self.offsets, pos=self.pos,
                      src=self.src, sel_bias=self.sel_bias, **common)
            loads = self.counts
        if c.bias_gamma > 0:
            # the loads of this step move the bias the next step selects with
            moe_update_bias(loads, c.ER, c.bias_gamma, self.sel_bias)

    def dispatch(self):
        c = self.cfg
        if c.mx:
            moe_dispatch(self.inp["x"], c.T, c.H, self.kr, self.src, self.R, None, self.xq,
                         self.xs, pos=self.pos)
            if self.xp is not None:  # GEMM1's input as the weight gradient dW1 needs it
                mx_dequantize(self.xq, self.xs, self.R, c.H, self.xp)
        else:
            moe_dispatch(self.inp["x"], c.T, c.H, self.kr, self.src, self.R, self.xp,
                         pos=self.pos)

    def experts(self):
        c, inp = self.cfg, self.inp
        if c.mx:
            moe_expert_ffn(MXFP8, self.xq, self.offsets, c.E, self.R, c.H, c.I, self.w1q,
                           self.w2q, self.y, xp_scales=self.xs, w1_scales=self.w1s,
                           w2_scales=self.w2s, gu_save=self.gu, h_save=self.h, ws=self.ffn_ws)
        else:
            moe_expert_ffn(BF16, self.xp, self.offsets, c.E, self.R, c.H, c.I, inp["w1"],
                           inp["w2"], self.y, gu_save=self.gu, h_save=self.h, ws=self.ffn_ws)
        if c.S:
            moe_expert_ffn(BF16, inp["x"], None, c.S, c.T, c.H, c.Is, inp["ws1"], inp["ws2"],
                           self.ys, gu_save=self.gus, h_save=self.hs, ws=self.sh_ws)

    def combine(self):
        c = self.cfg
        moe_combine(self.y, self.pos, self.w, c.T, self.kr, c.H, self.R, self.out, self.ys,
                    c.S)

    def forward(self):
        if self.ring:
            return self.forward_ring()
        self.route()
        self.dispatch()
        self.experts()
        self.combine()
        return self.out

    # ------------------------------------------------------------------ one launch
    def forward_fused(self):
        """The same forward as forward(), as one kernel launch (moe_layer_forward).
        BF16, unstreamed layers; outputs are bit-identical to forward()'s."""
        c, inp = self.cfg, self.inp
        if self.ring or c.mx:
            raise ValueError("the single-launch forward runs the unstreamed BF16 layer")
        if c.local_share and c.bias_gamma > 0:
            raise ValueError("the single-launch forward does not count the router's global "
                             "loads of a local share")
        if not hasattr(self, "fused"):
            self.fused = fwd_args(
                T=c.T, H=c.H, E=c.E, k=self.kr, I=c.I, S=c.S, Is=c.Is, E_router=c.ER,
                score=c.score, n_groups=c.n_groups, topk_groups=c.topk_groups,
                renorm=c.renorm, route_scale=c.route_scale, sel_bias=self.sel_bias,
                x=inp["x"], w_router=inp.get("w_router") if c.router_proj else None,
                logits=self.logits, idx_in=inp["idx_local"] if c.local_share else None,
                w1=inp["w1"], w2=inp["w2"], ws1=inp.get("ws1") if c.S else None,
                ws2=inp.get("ws2") if c.S else None, idx=self.idx, w=self.w, s_sel=self.s_sel,
                counts=self.counts, offsets=self.offsets, pos=self.pos, src=self.src,
                xp=self.xp, gu=self.gu, h=self.h, y=self.y, gus=self.gus if c.S else None,
                hs=self.hs if c.S else None, ys=self.ys, out=self.out)
            self.fused_ws = _e((max(layer_forward_workspace_size(self.fused), 256),),
                               torch.uint8, self.dev)
        moe_layer_forward(self.fused, self.fused_ws)
        if c.bias_gamma > 0:
            moe_update_bias(self.counts, c.ER, c.bias_gamma, self.sel_bias)
        return self.out

    # ------------------------------------------------------------------ HIP graph
    def capture(self, backward: bool = False):
        """One step of this layer -- the forward (per-step calls, or the ring's passes) and,
        with backward=True, the backward -- captured as a HIP graph over the layer's buffers.
        Replaying it reruns every launch of the step without host work between them.  The
        library allocates, frees and synchronises nothing and clears its own counters with
        kernels, so the calls capture as they run.  Returns the torch.cuda.CUDAGraph."""
        def step():
            self.forward()
            if backward:
                self.backward()

        side = torch.cuda.Stream(device=self.dev)  # default priority
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            step()  # first calls (per-device set-up of the library) outside the capture
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        return g

    # ------------------------------------------------------------------ macrobatch ring
    def _route_minibatch(self, a, b):
        # the selection alone (idx, w, s_sel of the minibatch's tokens): the rows are permuted
        # per pass, over the pass's minibatches, below
        c = self.cfg
        moe_route(self.logits[a:b], b - a, c.E, c.k, idx=self.idx[a:b], w=self.w[a:b],
                  s_sel=self.s_sel[a:b], counts=None, offsets=None, pos=None, src=None,
                  score=c.score, n_groups=c.n_groups, topk_groups=c.topk_groups,
                  renorm=c.renorm, route_scale=c.route_scale, ws=self.route_ws)

    def forward_ring(self):
        c, inp = self.cfg, self.inp
        T, H, E, I, k, mb = c.T, c.H, c.E, c.I, self.kr, self.mb
        x = inp["x"]
        for p in range(self.passes):
            t0 = p * self.pass_tokens
            t1 = min(T, t0 + self.pass_tokens)
            Tp, Rp = t1 - t0, (t1 - t0) * k
            # route every minibatch of the pass on its own
            for a in range(t0, t1, mb):
                self._route_minibatch(a, min(t1, a + mb))
            # the pass's rows into the ring slots: permutation, dispatch, one GEMM pass
            moe_route(None, Tp, E, k, idx_in=self.idx[t0:t1], counts=self.counts[p],
                      offsets=self.offsets[p], pos=self.pos[t0:t1], src=self.src[p],
                      ws=self.route_ws)
            r0 = (p if self.has_bwd else 0) * self.pass_rows
            xp, y = self.xp[r0:r0 + Rp], self.y[r0:r0 + Rp]
            moe_dispatch(x[t0:t1], Tp, H, k, self.src[p], Rp, xp, pos=self.pos[t0:t1])
            moe_expert_ffn(BF16, xp, self.offsets[p], E, Rp, H, I, inp["w1"], inp["w2"], y,
                           gu_save=None if self.gu is None else self.gu[r0:r0 + Rp],
                           h_save=self.h[r0:r0 + Rp], ws=self.ffn_ws)
            ys = None
            if c.S:
                ys = self.ys[0, t0:t1]
                moe_expert_ffn(BF16, x[t0:t1], None, 1, Tp, H, c.Is, inp["ws1"], inp["ws2"], ys,
                               gu_save=None if self.gus is None else self.gus[0, t0:t1],
                               h_save=self.hs[0, t0:t1], ws=self.sh_ws)
            # combine one minibatch at a time
            for a in range(t0, t1, mb):
                b = min(t1, a + mb)
                moe_combine(y, self.pos[a:b], self.w[a:b], b - a, k, H, Rp, self.out[a:b],
                            None if ys is None else self.ys[0, a:b], c.S)
        return self.out

    def backward(self):
        moe_backward(self.bargs, self.bwd_ws)
        return self.dx
