"""Seeded synthetic inputs for the mixture-of-experts layer workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and benchmark.
It holds no arithmetic of the layer: only the workload sizes, random draws, and the
rounding of those draws to bf16 storage.  Every random draw of a workload is keyed by
(seed, tensor id, sub-stream), so any one expert's weights can be regenerated alone.

Workloads follow the DeepSeek-V3-type layer that the pages name (pulsen.vercel.app,
"Cursor åpner megakernelen som ga 41 prosent flere tokens i sekundet", ¶6) at the
per-GPU share they measure (aiexpert.news, "Megakernels are dead and back…", ¶4:
expert-parallel degree 64, 2048 tokens per GPU).  The sizes of each workload are below.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

# Tensor ids: the second element of every seed key.
TID = dict(x=1, w_router=2, w1=3, w2=4, ws1=5, ws2=6, logits=7, dout=8,
           dirichlet=9, local_idx=10, outlier=11, zipf_perm=12, gumbel=13)

SOFTMAX, SIGMOID = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # source tokens
    H: int                 # hidden size
    E: int                 # routed experts on this GPU
    k: int                 # experts per token
    I: int                 # expert intermediate size
    S: int = 0             # shared experts
    Is: int = 0            # shared-expert intermediate size
    score: int = SOFTMAX
    renorm: bool = True
    route_scale: float = 1.0
    n_groups: int = 1
    topk_groups: int = 1
    E_router: int = 0      # experts the router scores over (0: same as E)
    local_share: bool = False   # routed rows are one GPU's share of a larger layer
    R_share: int = 0       # routed rows of that share
    router_proj: bool = False   # logits come from a router projection of x
    backward: bool = True
    mx: bool = False       # MXFP8 forward
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    zipf_s: float = 0.0    # >0: logits biased so expert loads follow Zipf(s)
    minibatch: int = 0     # >0: tokens stream through a ring in minibatches of this size
    x_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0

    @property
    def ER(self) -> int:
        return self.E_router or self.E

    @property
    def R(self) -> int:
        return self.R_share if self.local_share else self.T * self.k

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def fwd_flops(self) -> float:
        """Algorithmic forward flops: 6*H*I per routed row, 6*H*Is per shared row."""
        return 6.0 * self.H * self.I * self.R + 6.0 * self.H * self.Is * self.S * self.T


WORKLOADS = {
    # Tiny layer, forward only: router projection, softmax top-2 with renormalised weights.
    "tiny_t128": Workload("tiny_t128", T=128, H=256, E=8, k=2, I=512, router_proj=True,
                          backward=False),
    # Mid-size layer: softmax top-6 of 64, two shared experts.
    "mid_t2048": Workload("mid_t2048", T=2048, H=2048, E=64, k=6, I=1408, S=2, Is=1408),
    # DeepSeek-V3-shaped one-GPU share at expert-parallel degree 64: 4 local experts
    # receive 16384 routed rows from 2048 source tokens (sigmoid top-8 of 256 routing).
    "dsv3_ep64": Workload("dsv3_ep64", T=2048, H=7168, E=4, k=8, I=2048, score=SIGMOID,
                          E_router=256, local_share=True, R_share=16384),
    # Same shapes, MXFP8 forward, with 0.1% of activation channels scaled by 20.
    "dsv3_ep64_mxfp8": Workload("dsv3_ep64_mxfp8", T=2048, H=7168, E=4, k=8, I=2048,
                                score=SIGMOID, E_router=256, local_share=True,
                                R_share=16384, backward=False, mx=True,
                                outlier_frac=0.001, outlier_scale=20.0),
    # Full local 256-expert layer, Zipf(1.2)-skewed loads, group-limited sigmoid top-8
    # (8 groups, top-4 groups), one shared expert, minibatches of 512 through a ring.
    "dsv3_e256_zipf": Workload("dsv3_e256_zipf", T=8192, H=7168, E=256, k=8, I=2048, S=1,
                               Is=2048, score=SIGMOID, n_groups=8, topk_groups=4,
                               zipf_s=1.2, minibatch=512),
}


# ----------------------------------------------------------------------------- draws
def rng(wl: Workload, name: str, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([wl.seed, TID[name], sub])


def _torch_seed(wl: Workload, name: str, sub: int) -> int:
    ss = np.random.SeedSequence([wl.seed, TID[name], sub])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


def normal_bf16(wl: Workload, name: str, sub: int, shape, std: float, device="cpu",
                channel_scale: torch.Tensor | None = None) -> torch.Tensor:
    """N(0, std) drawn in fp32 with a seeded generator on `device`, rounded RNE to bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(wl, name, sub))
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    if channel_scale is not None:
        t.mul_(channel_scale.to(device))
    return t.to(torch.bfloat16)


def expert_weights(wl: Workload, device="cpu", shared: bool = False):
    """Stacked expert weights: w1 [E, 2I, H] (gate rows, then up rows), w2 [E, H, I]."""
    n, I, n1, n2 = (wl.S, wl.Is, "ws1", "ws2") if shared else (wl.E, wl.I, "w1", "w2")
    w1 = torch.empty(n, 2 * I, wl.H, dtype=torch.bfloat16, device=device)
    w2 = torch.empty(n, wl.H, I, dtype=torch.bfloat16, device=device)
    for e in range(n):
        w1[e] = normal_bf16(wl, n1, e, (2 * I, wl.H), wl.w_std, device)
        w2[e] = normal_bf16(wl, n2, e, (wl.H, I), wl.w_std, device)
    return w1, w2


def outlier_channels(wl: Workload) -> np.ndarray:
    n = int(round(wl.outlier_frac * wl.H))
    return np.sort(rng(wl, "outlier").choice(wl.H, size=n, replace=False)) if n else \
        np.zeros(0, np.int64)


def tokens(wl: Workload, device="cpu") -> torch.Tensor:
    scale = None
    ch = outlier_channels(wl)
    if len(ch):
        s = torch.ones(wl.H)
        s[torch.from_numpy(ch)] = wl.outlier_scale
        scale = s
    return normal_bf16(wl, "x", 0, (wl.T, wl.H), wl.x_std, device, channel_scale=scale)


def router_logits(wl: Workload) -> np.ndarray:
    """fp32 router logits [T, E_router].

    Zipf workloads: popularity p_e ∝ rank(e)^-s over a seeded permutation of the experts,
    logits ln p_e + Gumbel(0,1), so that the top-1 choice is exactly Zipf-distributed.
    Otherwise N(0,1).
    """
    T, E = wl.T, wl.ER
    if wl.zipf_s > 0:
        perm = rng(wl, "zipf_perm").permutation(E)
        rank = np.empty(E, np.int64)
        rank[perm] = np.arange(1, E + 1)
        p = rank.astype(np.float64) ** (-wl.zipf_s)
        p /= p.sum()
        gum = rng(wl, "gumbel").gumbel(size=(T, E))
        return (np.log(p)[None, :] + gum).astype(np.float32)
    return rng(wl, "logits").standard_normal((T, E), dtype=np.float32)


def local_share_idx(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Local expert of every routed pair of a one-GPU share.

    Expert probabilities p ~ Dirichlet(2,...,2); counts c ~ Multinomial(R, p); the pairs,
    laid out token-major as [T, k], take a seeded shuffle of the multiset {e repeated c_e}.
    """
    g = rng(wl, "dirichlet")
    p = g.dirichlet(np.full(wl.E, 2.0))
    c = g.multinomial(wl.R, p)
    ids = np.repeat(np.arange(wl.E, dtype=np.int32), c)
    rng(wl, "local_idx").shuffle(ids)
    return ids.reshape(wl.T, wl.R // wl.T), c.astype(np.int32)


def make_inputs(wl: Workload, device="cpu", weights: bool = True) -> dict:
    """All inputs of one workload as tensors on `device` (bf16 storage as torch.bfloat16)."""
    inp = {"x": tokens(wl, device)}
    if wl.router_proj:
        inp["w_router"] = normal_bf16(wl, "w_router", 0, (wl.ER, wl.H), wl.w_std, device)
    else:
        inp["logits"] = torch.from_numpy(router_logits(wl)).to(device)
    if wl.local_share:
        li, c = local_share_idx(wl)
        inp["idx_local"] = torch.from_numpy(li).to(device)
        inp["counts_local"] = torch.from_numpy(c).to(device)
    if weights:
        inp["w1"], inp["w2"] = expert_weights(wl, device)
        if wl.S:
            inp["ws1"], inp["ws2"] = expert_weights(wl, device, shared=True)
    if wl.backward:
        inp["dout"] = normal_bf16(wl, "dout", 0, (wl.T, wl.H), 1.0, device)
    return inp


# ----------------------------------------------------------------------------- bf16 bits
def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor's bits."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
