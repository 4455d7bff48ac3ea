"""Per-phase cycle trace of the fused INT8/FP8 attention kernel (diagnostic).

Builds a separate copy of the library with SAGE_PHASE_TRACE=1 (the product
library is not touched), runs a dense workload's attention through it in a
child process, and prints, per group of four waves, the shader-clock cycles per
phase pair spent in the matrix phase (PV of the previous tile and QK^T of this
one), in the softmax phase, waiting at the barrier between the phases, waiting
at the barrier that ends a pair (after this wave's loads), and the schedule's
total. Level 2 adds, per work-group, the cycles before the schedule starts and
the epilogue's, and, from each work-group's entry and exit times on its compute
unit, the gap between consecutive work-groups there. The trace build stores its
counters over part of the output, so its output is not an attention result.

    python -m quantized_attention_channel_amd.phase_trace [--workload peak] [--causal 1] [--pv fp8] [--level 2]

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
def trace_paths(level: int):
    suffix = "" if level == 1 else str(level)
    return (os.path.join(PKG, "_trace", f"libsage_trace{suffix}.so"), os.path.join(PKG, "_trace", f"obj{suffix}"))


def build_trace_library(level: int = 1) -> str:
    import importlib.util
    spec = importlib.util.spec_from_file_location("_sage_build", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib, obj = trace_paths(level)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    return b.build(defines=(f"SAGE_PHASE_TRACE={level}",), lib=lib, obj=obj)


def _child(workload: str, causal: bool, pv: str, level: int) -> None:
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
    if w.d != 128:
        raise SystemExit("the trace stores its counters in d = 128 output rows; pick a d = 128 workload")
    o = plan.o.contiguous().view(torch.int32).reshape(w.B * w.Hq, w.N, w.d // 2)
    rows = o[:, ::256, :64].cpu().numpy().astype(np.uint32).astype(np.float64)   # [BH, work-groups, 64]
    tr = rows.reshape(rows.shape[0], rows.shape[1], 8, 8)
    out = {}
    for g in (0, 1):
        sl = tr[:, :, 4 * g:4 * g + 4, :]
        n = sl[..., 4].sum()
        out[f"group{g}"] = {"matrix": sl[..., 0].sum() / n, "softmax": sl[..., 1].sum() / n,
                            "phase_barrier_wait": sl[..., 2].sum() / n, "pair_barrier_wait": sl[..., 3].sum() / n,
                            "total": sl[..., 5].sum() / n, "pairs_per_wave": n / sl[..., 4].size,
                            "prologue_per_wg": sl[..., 6].mean(), "epilogue_per_wg": sl[..., 7].mean()}
    if level < 2:
        print(json.dumps({"workload": w.name, "causal": w.causal, "pv": pv, "level": level,
                          "per_pair_cycles": out}), flush=True)
        return
    # work-group timeline (wave 0): entry/exit on the 100 MHz clock and the compute unit
    info = o[:, 1::256, :5].cpu().numpy().astype(np.uint32).astype(np.uint64)
    entry = info[..., 0] | (info[..., 1] << np.uint64(32))
    exit_ = info[..., 2] | (info[..., 3] << np.uint64(32))
    cu = info[..., 4]
    wg = {"span_us": float((exit_.max() - entry.min()) / 100.0),
          "mean_wg_us": float((exit_ - entry).astype(np.float64).mean() / 100.0)}
    gaps = []
    for c in np.unique(cu):
        sel = cu == c
        order = np.argsort(entry[sel])
        en, ex = entry[sel][order].astype(np.int64), exit_[sel][order].astype(np.int64)
        gaps.extend((en[1:] - ex[:-1]).tolist())
    gaps = np.array(gaps, dtype=np.float64) / 100.0
    wg.update({"cus": int(len(np.unique(cu))), "wgs_per_cu": float(entry.size / len(np.unique(cu))),
               "gap_us_mean": float(gaps.mean()) if gaps.size else 0.0,
               "gap_us_p90": float(np.percentile(gaps, 90)) if gaps.size else 0.0})
    print(json.dumps({"workload": w.name, "causal": w.causal, "pv": pv, "level": level, "per_pair_cycles": out,
                      "work_groups": wg}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="peak")
    ap.add_argument("--causal", type=int, default=0)
    ap.add_argument("--pv", default="fp8")
    ap.add_argument("--level", type=int, default=1, choices=(1, 2),
                    help="2: also the cycles before and after the schedule and the work-group timeline "
                         "(its extra live values slow the phases a little)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-build", action="store_true", help="reuse an existing trace library")
    args = ap.parse_args()
    if args.child:
        _child(args.workload, bool(args.causal), args.pv, args.level)
        return
    lib = trace_paths(args.level)[0]
    if not (args.no_build and os.path.exists(lib)):
        lib = build_trace_library(args.level)
    env = dict(os.environ, SAGE_LIB_PATH=lib)
    r = subprocess.run([sys.executable, "-m", "quantized_attention_channel_amd.phase_trace", "--child",
                        "--workload", args.workload, "--causal", str(args.causal), "--pv", args.pv,
                        "--level", str(args.level)],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    sys.stderr.write(r.stderr[-4000:])
    if r.returncode != 0:
        raise SystemExit(r.returncode)
    res = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    print(f"# {res['workload']} causal={int(res['causal'])} pv={res['pv']} level={res['level']}: "
          "shader-clock cycles per phase pair")
    print("| group | matrix phase | softmax phase | wait, phase barrier | wait, pair barrier | total per pair | pairs per wave |")
    print("|---|---|---|---|---|---|---|")
    for g in (0, 1):
        d = res["per_pair_cycles"][f"group{g}"]
        print(f"| {g} | {d['matrix']:.0f} | {d['softmax']:.0f} | {d['phase_barrier_wait']:.0f} | "
              f"{d['pair_barrier_wait']:.0f} | {d['total']:.0f} | {d['pairs_per_wave']:.1f} |")
    if res["level"] < 2:
        return
    print()
    print("| group | cycles before the schedule (per work-group) | epilogue issue (per work-group) |")
    print("|---|---|---|")
    for g in (0, 1):
        d = res["per_pair_cycles"][f"group{g}"]
        print(f"| {g} | {d['prologue_per_wg']:.0f} | {d['epilogue_per_wg']:.0f} |")
    wg = res["work_groups"]
    print()
    print(f"work-groups: {wg['cus']} compute units, {wg['wgs_per_cu']:.1f} per unit, {wg['mean_wg_us']:.1f} us each "
          f"(entry to exit of wave 0), {wg['span_us']:.0f} us in all; gap between consecutive work-groups on a unit "
          f"{wg['gap_us_mean']:.2f} us mean, {wg['gap_us_p90']:.2f} us at the 90th percentile")


if __name__ == "__main__":
    main()
