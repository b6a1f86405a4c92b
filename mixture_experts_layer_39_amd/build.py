"""Build libmoe.so (the gfx950 HIP library behind include/moe.h) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["abi.hip", "route.hip", "rows.hip", "gemm.hip", "gemm_mx.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (they are never needed here)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit fused multiply-add: the routing keys follow a fixed sequence of IEEE
    # operations, each rounded once
    "-ffp-contract=off",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + FLAGS + (extra or []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    n_warn = sum(1 for l in errs.splitlines() if ": warning:" in l)
    if n_warn:
        # every warning is reported, so that a new one cannot go unnoticed
        print(f"hipcc: {n_warn} warning(s)", file=sys.stderr, flush=True)
        print(errs, file=sys.stderr, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
