"""Per-phase cycle trace of the fused INT8/FP8 attention kernel (diagnostic).

Builds a separate copy of the library with SAGE_PHASE_TRACE=1 (the product
library is not touched), runs a dense workload's attention through it in a
child process, and prints, per group of four waves, the shader-clock cycles per
phase pair spent in the matrix phase (PV of the previous tile and QK^T of this
one), in the softmax phase, waiting at the barrier between the phases, waiting
at the barrier that ends a pair (after this wave's loads), and the schedule's
total. The trace build stores its counters over part of the output, so its
output is not an attention result.

    python -m quantized_attention_channel_amd.phase_trace [--workload peak] [--causal 1] [--pv fp8]

Clock reads around a phase count the cycles its instructions take to issue;
the matrix work then drains under the barrier that follows, which is where the
other group's phase ends.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRACE_LIB = os.path.join(PKG, "_trace", "libsage_trace.so")
TRACE_OBJ = os.path.join(PKG, "_trace", "obj")


def build_trace_library() -> str:
    import importlib.util
    spec = importlib.util.spec_from_file_location("_sage_build", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    os.makedirs(os.path.dirname(TRACE_LIB), exist_ok=True)
    return b.build(defines=("SAGE_PHASE_TRACE=1",), lib=TRACE_LIB, obj=TRACE_OBJ)


def _child(workload: str, causal: bool, pv: str) -> None:
    """Runs under SAGE_LIB_PATH = the trace library; prints one JSON line."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bench
    import workloads as W
    w = bench.ALIASES.get(workload) or W.ALL[workload]
    w = w.with_(causal=causal)
    if w.layout != "HND":
        raise SystemExit("the trace reads its counters back in the HND layout; pick an HND workload")
    q, k, v = W.generate(w, device="cuda")
    plan = bench.Plan(w, pv, q, k, v)
    for _ in range(3):
        plan.quant()
        plan.attention()
    torch.cuda.synchronize()
    o = plan.o.contiguous().view(torch.int32).reshape(w.B * w.Hq, w.N, w.d // 2)
    rows = o[:, ::256, :64].cpu().numpy().astype(np.uint32).astype(np.float64)   # [BH, pairs, 64]
    tr = rows.reshape(rows.shape[0], rows.shape[1], 8, 8)
    out = {}
    for g in (0, 1):
        sl = tr[:, :, 4 * g:4 * g + 4, :]
        n = sl[..., 4].sum()
        out[f"group{g}"] = {"matrix": sl[..., 0].sum() / n, "softmax": sl[..., 1].sum() / n,
                            "phase_barrier_wait": sl[..., 2].sum() / n, "pair_barrier_wait": sl[..., 3].sum() / n,
                            "total": sl[..., 5].sum() / n, "pairs_per_wave": n / sl[..., 4].size}
    print(json.dumps({"workload": w.name, "causal": w.causal, "pv": pv, "per_pair_cycles": out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="peak")
    ap.add_argument("--causal", type=int, default=0)
    ap.add_argument("--pv", default="fp8")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-build", action="store_true", help="reuse an existing trace library")
    args = ap.parse_args()
    if args.child:
        _child(args.workload, bool(args.causal), args.pv)
        return
    lib = TRACE_LIB if args.no_build and os.path.exists(TRACE_LIB) else build_trace_library()
    env = dict(os.environ, SAGE_LIB_PATH=lib)
    r = subprocess.run([sys.executable, "-m", "quantized_attention_channel_amd.phase_trace", "--child",
                        "--workload", args.workload, "--causal", str(args.causal), "--pv", args.pv],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    sys.stderr.write(r.stderr[-4000:])
    if r.returncode != 0:
        raise SystemExit(r.returncode)
    res = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    print(f"# {res['workload']} causal={int(res['causal'])} pv={res['pv']}: shader-clock cycles per phase pair")
    print("| group | matrix phase | softmax phase | wait, phase barrier | wait, pair barrier | total per pair | pairs per wave |")
    print("|---|---|---|---|---|---|---|")
    for g in (0, 1):
        d = res["per_pair_cycles"][f"group{g}"]
        print(f"| {g} | {d['matrix']:.0f} | {d['softmax']:.0f} | {d['phase_barrier_wait']:.0f} | "
              f"{d['pair_barrier_wait']:.0f} | {d['total']:.0f} | {d['pairs_per_wave']:.1f} |")


if __name__ == "__main__":
    main()
