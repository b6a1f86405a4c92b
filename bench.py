"""Throughput of the deterministic MoE layer on one MI355X, with its roofline and a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole layer over one batch: routing (router top-k and the
expert-contiguous permutation), dispatch, the grouped-GEMM expert FFN, the weighted combine and,
for workloads with a backward, the BF16 backward of all of it.  Inputs are seeded synthetic
tensors already resident in HBM; every step runs through the HIP kernels of libmoe.so.

The default workload is the DeepSeek-V3-shaped one-GPU share at expert-parallel degree 64
(2048 source tokens per GPU, 4 local experts receiving 16384 routed rows, hidden 7168,
SwiGLU intermediate 2048), the per-GPU shape the pages measure their layer at.

Printed: ONE JSON line.  `value` is forward+backward tokens/s (source tokens per second of
wall time, K steps bracketed by device synchronisation).  `fwd_tokens_per_s` times forward-only
steps the same way.  `roofline` is for the kernel that takes the largest share of a step:
its algorithmic flops (or bytes) per launch over its average launch duration, measured with
HIP events the library records around each of its launches on the launch stream, over K more
steps run after the timed ones (the event records add gaps between launches, not kernel
time; `traced_ms_per_step` is the step time with them).
`cold_tokens_per_s` times the same steps one by one with cold caches (a 1 GiB read before each
step evicts L2 and the Infinity Cache).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd & fwd+bwd (1 GPU); grouped-GEMM MFMA % of peak"

# MI355X published peaks (dense)
PEAK_BF16_TFLOPS = 2500.0
PEAK_MXFP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0

GEMM_ROLES = {  # role -> (flops per routed row in units of H*I, MX)
    "gemm1_swiglu": (4, False), "gemm2_down": (2, False),
    "ffn_queue": (6, False),      # GEMM1 + SwiGLU and GEMM2 as one launch (tile queue)
    "bwd_down": (4, False),       # dh = dy W2 (+ SwiGLU backward) and dW2 = dy^T h
    "bwd_gate_up": (8, False),    # dXp = dGU W1 and dW1 = dGU^T Xp
    "mx_gemm1_swiglu": (4, True), "mx_gemm2_down": (2, True),
    "mx_bwd_down": (2, True),     # MXFP8 dgrad: dh = Q(dy) Q(W2^T)^T (+ SwiGLU backward)
    "mx_bwd_gate_up": (4, True),  # MXFP8 dgrad: dXp = Q(dGU) Q(W1^T)^T
    "wgrad_down": (2, False),     # dW2 = dy^T h alone (after MXFP8 dgrad)
    "wgrad_gate_up": (4, False),  # dW1 = dGU^T Xp alone
    "mx_bwd_down_wgrad": (4, True),     # MXFP8 dh (+ SwiGLU backward) and dW2 = Qt(dy)^T Qt(h)
    "mx_bwd_gate_up_wgrad": (8, True),  # MXFP8 dXp and dW1 = Qt(dGU)^T Qt(Xp)
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first; the clocks settle over the first tens of ms")
    ap.add_argument("--workload", default="dsv3_ep64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=48,
                    help="source tokens of the CPU-oracle sample")
    ap.add_argument("--all-configs", action=argparse.BooleanOptionalAction, default=True,
                    help="after the headline workload (dsv3_ep64), also measure the other "
                         "workloads and report them under \"configs\"")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed as a HIP graph (graph_ms_per_step)")
    ap.add_argument("--breakdown", action="store_true",
                    help="also print per-role times to stderr")
    ap.add_argument("--ring-depth", type=int, default=16,
                    help="minibatches per pass of the macrobatch ring (workloads that stream "
                         "tokens in minibatches)")
    ap.add_argument("--backward", action="store_true",
                    help="add the backward to a forward-only workload (MXFP8: MXFP8 dgrad)")
    ap.add_argument("--fused", action="store_true",
                    help="run each step's forward as one launch (moe_layer_forward)")
    ap.add_argument("--bias-gamma", type=float, default=0.0,
                    help="> 0: the sigmoid router's load-balancing bias is updated from the "
                         "step's loads with this speed (auxiliary-loss-free balancing)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="calibration run: only a plain device copy (read N MiB, write N MiB) "
                         "a few times, for scaling hardware byte counters; prints its size")
    ap.add_argument("--traffic-from", default="",
                    help="no GPU: condense rocprofv3 counter runs under this folder (subfolders "
                         "fetch/, write/, copy_fetch/, copy_write/) into profiles/hbm_traffic.json")
    return ap.parse_args()


# ----------------------------------------------------------------------------- algorithmic work
def role_work(wl, role: str, shared: bool) -> tuple[str, float]:
    """Algorithmic work of one launch of `role`: ("flop", n) or ("byte", n)."""
    H, I, R, T, k = wl.H, wl.I, wl.R, wl.T, (wl.R // wl.T if wl.T else wl.k)
    if shared:
        I, R = wl.Is, wl.T
    if role in GEMM_ROLES:
        return "flop", float(GEMM_ROLES[role][0]) * H * I * R
    bf = 2
    if role == "dispatch":          # unique source rows read once + every routed row written
        return "byte", float(T * H * bf + R * H * bf + R * 4)
    if role == "dispatch_mx":
        return "byte", float(T * H * bf + R * H + R * H // 32 + R * 4)
    if role == "combine":
        return "byte", float(R * H * bf + wl.S * T * H * bf + T * H * bf + T * k * 8)
    if role == "combine_bwd":
        if wl.mx:  # MXFP8 weight gradients: no dy rows, each row's source slot and weight
            return "byte", float(T * H * bf + R * H * bf + T * k * 12 + R * 8)
        return "byte", float(T * H * bf + 2 * R * H * bf + T * k * 12)
    if role == "unpermute":
        return "byte", float(R * H * bf + wl.S * T * H * bf + T * H * bf + T * k * 4)
    if role == "router_proj":       # x and the router weight read, fp32 logits written
        return "byte", float(T * H * bf + wl.ER * H * bf + T * wl.ER * 4)
    if role == "topk":
        return "byte", float(T * wl.ER * 4 + T * wl.k * 12)
    if role == "bias_update":       # loads read, bias read and written
        return "byte", float(wl.ER * 12)
    if role == "router_bwd":
        return "byte", float(T * wl.ER * 4 + T * wl.k * 16)
    if role == "mx_quantize_dy":    # bf16 dy read, codes and scales written
        return "byte", float(R * H * bf + R * H + R * H // 32)
    if role == "mx_quantize_dgu":
        return "byte", float(R * 2 * I * bf + R * 2 * I + R * 2 * I // 32)
    if role == "mx_quantize_tok_xp":  # xp's dispatch codes and scales in, codes and scales out
        return "byte", float(R * H + R * H // 32 + R * H + R * H // 32)
    if role == "mx_quantize_tok_dy":  # dy formed from dout (each token's row, the rows'
        # sources) and quantised along the tokens and along H in one pass
        return "byte", float(T * H * bf + R * 12 + 2 * (R * H + R * H // 32))
    if role == "mx_quantize_tok_dgu":  # bf16 dGU in, codes and scales along the tokens and 2I
        return "byte", float(R * 2 * I * bf + 2 * (R * 2 * I + R * 2 * I // 32))
    if role.startswith("mx_quantize_tok_"):  # a [R, C] bf16 operand in, codes and scales out
        C = {"h": I}[role[len("mx_quantize_tok_"):]]
        return "byte", float(R * C * bf + R * C + R * C // 32)
    if role == "mx_dequantize":     # xp codes and scales read, bf16 written (and h after GEMM2)
        return "byte", float(R * H + R * H // 32 + R * H * bf)
    return "byte", 0.0


def gemm_bytes(wl, role: str, shared: bool) -> float:
    """Algorithmic HBM bytes of one launch of a BF16 grouped-GEMM role: every operand, weight
    and result it must read or write once (bf16), for the routed experts or (shared) the
    shared experts.  0 for roles without a byte model (the MXFP8 products)."""
    H, I, R, E = wl.H, wl.I, wl.R, wl.E
    if shared:
        I, R, E = wl.Is, wl.T, wl.S
    b = 2.0
    xp, h, gu, w = R * H * b, R * I * b, R * 2 * I * b, E * H * I * b  # w: one of W1/2 halves
    gu_save = gu if wl.backward else 0.0
    return {
        "gemm1_swiglu": xp + 2 * w + h + gu_save,          # Xp, W1 in; h (and g|u) out
        "gemm2_down": h + w + xp,                          # h, W2 in; y out
        "ffn_queue": xp + 2 * w + 2 * h + w + xp + gu_save,  # both products (h out and in)
        "bwd_down": xp + w + gu + gu + h + w,              # dy, W2, g|u, h in; dGU, dW2 out
        "bwd_gate_up": gu + 2 * w + xp + xp + 2 * w,       # dGU, W1, Xp in; dXp, dW1 out
    }.get(role, 0.0)


def step_work(wl, role: str) -> tuple[str, float]:
    """Algorithmic work of `role` over one step: the routed experts' share plus, for the BF16
    GEMMs, the shared experts' (each of them runs on every source token)."""
    kind, work = role_work(wl, role, shared=False)
    if role in GEMM_ROLES and not GEMM_ROLES[role][1] and wl.S and not wl.local_share:
        work += wl.S * role_work(wl, role, shared=True)[1]
    return kind, work


def roofline_of(wl, role: str, ms_per_step: float, launches: float, traffic) -> dict:
    """Roofline of `role`: its algorithmic work per step over its measured time per step (the
    sum of its launch durations), and the same per launch.  A BF16 GEMM role is held against
    the bound that takes longer at the published peaks -- its flops at the MFMA peak or its
    algorithmic bytes at the HBM peak -- and reports its fraction of both."""
    kind, work = step_work(wl, role)
    per_launch_ms = ms_per_step / launches
    common = {"work_per_launch": work / launches, "avg_launch_ms": round(per_launch_ms, 4),
              "launches_per_step": launches}
    if kind == "flop":
        peak = PEAK_MXFP8_TFLOPS if GEMM_ROLES[role][1] else PEAK_BF16_TFLOPS
        ach = work / (ms_per_step * 1e-3) / 1e12
        nbytes = gemm_bytes(wl, role, False)
        if nbytes and wl.S and not wl.local_share:
            nbytes += gemm_bytes(wl, role, True)
        if nbytes:
            gbs = nbytes / (ms_per_step * 1e-3) / 1e9
            common.update(mfma_frac=round(ach / peak, 4), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                          bytes_per_launch=nbytes / launches)
            if nbytes / (PEAK_HBM_GBS * 1e9) > work / (peak * 1e12):
                return {"kernel": role, "bound": "hbm", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic, **common}
        return {"kernel": role, "bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic, **common}
    ach = work / (ms_per_step * 1e-3) / 1e9
    return {"kernel": role, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, **common}


def kernel_source_digest() -> str:
    """Digest of the HIP sources; stored HBM-traffic counts are valid only for this digest."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_39_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, role: str, ring_depth=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    summary is missing, was taken on different kernel sources, or in another launch
    configuration (a ring layer's launches move different bytes at another ring depth)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_digest") != kernel_source_digest():
        return None
    if d.get("ring_depth", {}).get(workload) != ring_depth:
        return None
    ent = d.get("workloads", {}).get(workload, {}).get(role)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- HBM traffic
COPY_KERNEL_HINT = "MulFunctor"   # torch's elementwise multiply: the calibration copy


def role_of_symbol(sym: str) -> str:
    """Launch role of a kernel symbol as rocprofv3 names it (demangled)."""
    base = sym.split("(")[0].split("<")[0].strip()
    base = base.split(" ")[-1].split("::")[-1]
    if base.endswith("_kernel"):
        base = base[: -len("_kernel")]
    return {"count": "perm_count", "scan": "perm_scan", "rank": "perm_rank"}.get(base, base)


def _counter_means(folder: str, counter: str) -> dict[str, tuple[int, float]]:
    """kernel symbol -> (dispatches, mean counter value) over every counter CSV in folder."""
    import csv
    import glob
    acc: dict[str, list[float]] = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def write_traffic(folder: str, workload: str, copy_mib: int, ring_depth=None) -> None:
    """profiles/hbm_traffic.json from four rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch) of the layer's kernels, each scaled by the ratio of the known size of a plain
    copy to what the same counter reads for it."""
    known_kib = copy_mib * 1024.0
    scale = {}
    for ctr, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        m = {k: v for k, v in _counter_means(os.path.join(folder, sub), ctr).items()
             if COPY_KERNEL_HINT in k}
        if not m:
            raise SystemExit(f"no copy kernel ({COPY_KERNEL_HINT}) in {sub}")
        _, kib = max(m.values(), key=lambda t: t[1])
        scale[ctr] = known_kib / kib
    fetch = _counter_means(os.path.join(folder, "fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(folder, "write"), "WRITE_SIZE")
    roles = {}
    for sym in sorted(set(fetch) | set(write)):
        if COPY_KERNEL_HINT in sym or "moe::" not in sym:
            continue
        role = role_of_symbol(sym)
        n, fk = fetch.get(sym, (0, 0.0))
        _, wk_ = write.get(sym, (0, 0.0))
        fb, wb = fk * 1024 * scale["FETCH_SIZE"], wk_ * 1024 * scale["WRITE_SIZE"]
        roles[role] = {"symbol": sym, "dispatches": n, "fetch_kib_raw": round(fk, 1),
                       "write_kib_raw": round(wk_, 1), "fetch_bytes": round(fb),
                       "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    workloads, depths = {}, {}
    try:  # counts of other workloads taken on the same sources stay
        with open(path) as fh:
            prev = json.load(fh)
        if prev.get("kernel_source_digest") == kernel_source_digest():
            workloads = prev.get("workloads", {})
            depths = prev.get("ring_depth", {})
    except (OSError, ValueError):
        pass
    workloads[workload] = roles
    depths[workload] = ring_depth
    out = {"kernel_source_digest": kernel_source_digest(),
           "counters": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (separate runs), "
                       "mean KiB per dispatch",
           "copy_calibration": {"kernel": COPY_KERNEL_HINT, "mib": copy_mib,
                                "fetch_scale": round(scale["FETCH_SIZE"], 4),
                                "write_scale": round(scale["WRITE_SIZE"], 4)},
           "ring_depth": depths,
           "workloads": workloads}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"| role | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes/launch (scaled) |")
    print(f"|---|---|---|---|---|")
    for r, e in roles.items():
        print(f"| {r} | {e['dispatches']} | {e['fetch_kib_raw']} | {e['write_kib_raw']} | "
              f"{e['hbm_bytes_per_launch']:.4g} |")
    print(f"copy scales: fetch {scale['FETCH_SIZE']:.4f} write {scale['WRITE_SIZE']:.4f}; "
          f"wrote {path}")


def cold_ms_per_call(f, calls: int, flush_mib: int = 1024) -> float:
    """Average device time of f() with cold caches.  Before each call a reduction reads
    flush_mib MiB (four times the 256 MB Infinity Cache, and far beyond the L2s), which
    writes back and evicts whatever the previous call left there, and leaves only clean lines
    of the flush buffer behind.  HIP events on the launch stream bracket f() alone; the host
    never waits inside the loop, so the launches queue ahead of the device."""
    import torch
    # float32: the reduction reads the buffer as it is (an integer sum would widen it first)
    buf = torch.ones(flush_mib << 18, dtype=torch.float32, device="cuda:0")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    f()
    torch.cuda.synchronize()
    for i in range(calls):
        buf.sum()
        starts[i].record()
        f()
        ends[i].record()
    torch.cuda.synchronize()
    ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / calls
    del buf
    return ms


def copy_calibration(mib: int) -> None:
    """A plain device copy of known size (read mib MiB, write mib MiB), five times."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "read_bytes": n * 4, "write_bytes": n * 4}), flush=True)


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, inp, n_tokens: int) -> dict:
    """The CPU oracle (fp64 plain loops) on the first n_tokens source tokens of the workload,
    forward (+ backward when the workload has one); tokens/s of that sample.  Layers with
    many experts keep only the weights of the experts the sample's tokens select (the
    oracle's own selection of those tokens; the tokens then reach them as a local share)."""
    import numpy as np
    import oracle as orc
    import workloads as wk
    n = min(n_tokens, wl.T)
    p = dict(x=wk.bf16_bits(inp["x"][:n]), k=wl.k, score=wl.score, renorm=wl.renorm,
             route_scale=wl.route_scale, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
             mx=wl.mx)
    if "w_router" in inp:
        p["w_router"] = wk.bf16_bits(inp["w_router"])
    else:
        p["logits"] = inp["logits"][:n].cpu().numpy()
    experts = "the full expert weights"
    if "idx_local" in inp:
        p["idx_local"] = inp["idx_local"][:n].cpu().numpy()
        p["w1"], p["w2"] = wk.bf16_bits(inp["w1"]), wk.bf16_bits(inp["w2"])
    elif wl.E > 64:
        idx, _ = orc.route_select(p["logits"], wl.k, wl.score, wl.n_groups, wl.topk_groups)
        used = np.unique(idx)
        p["idx_local"] = np.searchsorted(used, idx).astype(np.int32)
        sel = torch_index(used).to(inp["w1"].device)
        p["w1"], p["w2"] = wk.bf16_bits(inp["w1"][sel]), wk.bf16_bits(inp["w2"][sel])
        experts = f"the weights of the {len(used)} experts they select"
    else:
        p["w1"], p["w2"] = wk.bf16_bits(inp["w1"]), wk.bf16_bits(inp["w2"])
    if wl.S:
        p["ws1"], p["ws2"] = wk.bf16_bits(inp["ws1"]), wk.bf16_bits(inp["ws2"])
    dout = wk.bf16_bits(inp["dout"][:n]) if wl.backward else None
    orc.lib()
    t0 = time.perf_counter()
    r = orc.layer_forward(p)
    if wl.backward:
        orc.layer_backward(p, r, dout)
    dt = time.perf_counter() - t0
    rows = int(p["idx_local"].size) if "idx_local" in p else n * wl.k
    what = "forward+backward" if wl.backward else "forward"
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": orc.threads(),
            "cpu": _cpu_model(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {n} of {wl.T} source tokens ({rows} routed rows) with "
                      f"{experts}, oracle {what} in fp64"}


def torch_index(a):
    import torch
    return torch.from_numpy(a.astype("int64"))


def _cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


# ----------------------------------------------------------------------------- main
def main():
    a = parse()
    if a.traffic_from:
        import workloads as wk
        write_traffic(a.traffic_from, a.workload, a.copy_mib or 1024,
                      a.ring_depth if wk.WORKLOADS[a.workload].minibatch else None)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the layer on one GPU; the expert-parallel "
              "path across GPUs is not implemented (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import mixture_experts_layer_39_amd as moe
    import workloads as wk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_mib:
        copy_calibration(a.copy_mib)
        return
    moe.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    wl = wk.WORKLOADS[a.workload]
    if a.backward and not wl.backward:
        wl = wl.scaled(backward=True)
    head = measure(wl, a, ring_depth=a.ring_depth, steps=a.steps, warmup=a.warmup,
                   fused=a.fused, bias_gamma=a.bias_gamma, headline=True,
                   cpu_tokens=None if a.no_cpu_baseline else a.cpu_tokens)
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "traced_ms_per_step": head["traced_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8" if wl.mx else "bf16",
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": head["config"],
    }
    for key in ("fwd_tokens_per_s", "fwd_ms_per_step", "step_tflops", "fwd_tflops",
                "cold_tokens_per_s", "cold_ms_per_step", "cold_fwd_ms_per_step",
                "fused_fwd_ms_per_step", "fused_fwd_tokens_per_s", "graph_ms_per_step",
                "graph_tokens_per_s", "roofline", "breakdown",
                "cpu_baseline"):
        out[key] = head.get(key)
    if a.all_configs and a.workload == "dsv3_ep64" and not a.fused:
        # the other workloads, each measured the same way (fewer warm-up steps: the GPU is
        # warm by now), compactly: throughput, the dominant kernel's roofline and a CPU sample
        extra = {}
        plan = [("tiny_t128", "tiny_t128", {}), ("mid_t2048", "mid_t2048", {}),
                ("dsv3_ep64_mxfp8", "dsv3_ep64_mxfp8", {}),
                ("dsv3_ep64_mxfp8_bwd", "dsv3_ep64_mxfp8", {"backward": True}),
                ("dsv3_e256_zipf", "dsv3_e256_zipf", {"ring_depth": a.ring_depth}),
                ("dsv3_e256_zipf_ring4", "dsv3_e256_zipf", {"ring_depth": 4})]
        cpu_tokens = {"tiny_t128": 128, "mid_t2048": 16, "dsv3_ep64_mxfp8": 48,
                      "dsv3_e256_zipf": 4}
        for key, name, opt in plan:
            w = wk.WORKLOADS[name]
            if opt.get("backward"):
                w = w.scaled(backward=True)
            ct = None
            if not a.no_cpu_baseline and key in cpu_tokens:
                ct = cpu_tokens[key]
            rec = measure(w, a, ring_depth=opt.get("ring_depth", a.ring_depth),
                          steps=a.steps, warmup=min(a.warmup, 5), fused=False, bias_gamma=0.0,
                          headline=False, cpu_tokens=ct)
            extra[key] = rec
            print(f"bench: {key} {rec['ms_per_step']} ms/step", file=sys.stderr, flush=True)
        out["configs"] = extra
    print(json.dumps(out), flush=True)


def measure(wl, a, *, ring_depth, steps, warmup, fused, bias_gamma, headline, cpu_tokens):
    """One workload: K untimed-warm-up, K timed and K traced steps; the record of its
    throughput, the dominant kernel's roofline, and (headline) the cold-cache and per-role
    figures.  The layer's buffers are freed before returning."""
    import torch
    import workloads as wk
    import mixture_experts_layer_39_amd as moe
    from mixture_experts_layer_39_amd.layer import LayerCfg, MoELayer

    dev = "cuda:0"
    inp = wk.make_inputs(wl, device=dev)
    ring = dict(minibatch=wl.minibatch, ring_depth=ring_depth) if wl.minibatch else {}
    lcfg = LayerCfg.from_workload(wl)
    lcfg.bias_gamma = bias_gamma
    layer = MoELayer(lcfg, inp, dev, backward=wl.backward, **ring)
    can_fuse = not wl.mx and not layer.ring and not (wl.local_share and bias_gamma > 0)
    if fused and not can_fuse:
        print("--fused runs the unstreamed BF16 layer only", file=sys.stderr)
        sys.exit(2)
    fwd = layer.forward_fused if fused else layer.forward

    def step():
        fwd()
        if wl.backward:
            layer.backward()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed: K whole steps (the throughput), without instrumentation
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / steps

    # traced: K more identical steps with per-launch HIP events recorded by the library on
    # each launch's stream (the kernel durations of the roofline and the breakdown).  The
    # event records add gaps between launches (about 0.1 ms per step at the EP-64 share) but
    # not kernel time, so the throughput comes from the untraced steps above.
    moe.trace_begin(max(512, 512 * steps))
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    recs = moe.trace_end()
    traced_ms_step = (t3 - t2) * 1e3 / steps

    # forward-only steps, untraced: the per-step calls, and (where it applies) the forward
    # as one launch
    def time_fwd(f):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for _ in range(steps):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - f0) * 1e3 / steps

    fwd_ms = time_fwd(layer.forward) if wl.backward or fused else ms_step
    fused_ms = time_fwd(layer.forward_fused) if can_fuse else None

    # the same whole step replayed as a HIP graph (every launch of the step, no host work
    # between them), untraced
    graph_ms = None
    if not fused and a.graph:
        g = layer.capture(backward=wl.backward)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g0) * 1e3 / steps
        del g

    # per-role statistics over the traced steps
    roles: dict[str, list[float]] = {}
    for name, ms in recs:
        roles.setdefault(name, []).append(ms)
    per_step = {r: sum(v) / steps for r, v in roles.items()}
    dominant = max(per_step, key=per_step.get)
    roof = roofline_of(wl, dominant, per_step[dominant], len(roles[dominant]) / steps,
                       measured_traffic(wl.name, dominant,
                                        ring_depth if wl.minibatch else None))

    flops_fwd = wl.fwd_flops()
    flops_step = flops_fwd * (3.0 if wl.backward else 1.0)
    cfg = {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k, "I": wl.I,
           "routed_rows": wl.R, "S": wl.S, "Is": wl.Is, "E_router": wl.ER,
           "score": "sigmoid" if wl.score == wk.SIGMOID else "softmax",
           "n_groups": wl.n_groups, "topk_groups": wl.topk_groups,
           "precision": "mxfp8" if wl.mx else "bf16", "backward": wl.backward,
           "parallelism": "none (one GPU's share)"}
    if layer.ring:
        cfg.update(minibatch=layer.mb, ring_depth=layer.D, ring_passes=layer.passes)
    if bias_gamma > 0:
        cfg.update(bias_gamma=bias_gamma)
    if fused:
        cfg.update(forward="one launch")
    if wl.mx and wl.backward:
        cfg.update(backward_precision="mxfp8 dgrad and weight gradients")
    rec = {
        "config": cfg,
        "tokens_per_s": round(wl.T * steps / elapsed, 1),
        "ms_per_step": round(ms_step, 4),
        "traced_ms_per_step": round(traced_ms_step, 4),
        "fwd_tokens_per_s": round(wl.T / (fwd_ms * 1e-3), 1),
        "fwd_ms_per_step": round(fwd_ms, 4),
        "step_tflops": round(flops_step / (ms_step * 1e-3) / 1e12, 1),
        "fwd_tflops": round(flops_fwd / (fwd_ms * 1e-3) / 1e12, 1),
        "fused_fwd_ms_per_step": round(fused_ms, 4) if fused_ms else None,
        "fused_fwd_tokens_per_s": round(wl.T / (fused_ms * 1e-3), 1) if fused_ms else None,
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms else None,
        "graph_tokens_per_s": round(wl.T / (graph_ms * 1e-3), 1) if graph_ms else None,
        "roofline": roof,
    }
    if layer.ring or wl.E > 8:
        c = layer.counts.view(-1, wl.E).sum(0).cpu()
        rec["loads"] = {"min": int(c.min()), "median": int(c.median()), "max": int(c.max())}
    if headline:
        cold_ms = cold_ms_per_call(step, steps)
        cold_fwd_ms = cold_ms_per_call(layer.forward, steps)
        rec.update(cold_tokens_per_s=round(wl.T / (cold_ms * 1e-3), 1),
                   cold_ms_per_step=round(cold_ms, 4), cold_fwd_ms_per_step=round(cold_fwd_ms, 4))
        breakdown = {}
        for r in sorted(per_step, key=per_step.get, reverse=True):
            n = len(roles[r]) / steps
            ent = {"launches_per_step": n, "ms_per_step": round(per_step[r], 4),
                   "share": round(per_step[r] / traced_ms_step, 4)}
            kind, work = step_work(wl, r)
            if kind == "flop":
                ent["tflops"] = round(work / (per_step[r] * 1e-3) / 1e12, 1)
            elif work and n == 1:
                ent["gbs"] = round(work / (per_step[r] * 1e-3) / 1e9, 1)
            breakdown[r] = ent
        rec["breakdown"] = breakdown
        if a.breakdown:
            for r, e in breakdown.items():
                print(f"  {r:22s} {e}", file=sys.stderr)
    rec["cpu_baseline"] = cpu_baseline(wl, inp, cpu_tokens) if cpu_tokens else None
    del layer, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


if __name__ == "__main__":
    main()
