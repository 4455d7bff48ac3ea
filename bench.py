#!/usr/bin/env python3
"""Attention TOPS of the quantised-attention forward hot path on one MI355X.

A *step* is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM: K channel statistics and smoothing, per-block
INT8 Q/K, per-channel e4m3 V, and the fused attention kernel (INT8 QK^T,
dequantisation, online softmax, P to e4m3, PV with two-level accumulation,
epilogue). It is issued through the C ABI as sage_quant_qk + sage_quant_v +
sage_attn_fwd_codes -- exactly the kernels sage_attn_fwd enqueues -- so that
HIP events can bracket the attention kernel inside every timed step.

value        = 4*B*H*N^2*d (halved for causal) / wall time per step   [TOPS]
roofline     = the attention kernel alone: the same counted operations / its
               mean event-timed duration, against the dense INT8/FP8 MFMA peak
cpu_baseline = the CPU oracle on a bounded sample of the same workload.

Default workload: B=1, H=32, N=32768, d=128, fp16, non-causal, PV in e4m3 (the
long-sequence peak workload), per-block Q/K scales; the causal variant, the per-thread-scale variant and a
packed variable-length serving mix (16 causal GQA sequences of 256-16384
tokens, one sage_attn_fwd_varlen call per step) are reported alongside.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "attention TOPS (4·B·H·N²·d/t) at N=32K d=128 + % of INT8/FP8 MFMA peak"
PEAK_TOPS = 5000.0            # MI355X dense INT8 and dense FP8 MFMA peak (5.0 POP/s each)
PEAK_FP4_TOPS = 10100.0       # MI355X dense FP4 (and FP6) MFMA peak, 10.1 PFLOP/s
PEAK_HBM_GBS = 8000.0
ALIASES = {"tiny": W.TINY, "mid": W.MID_OUTLIER, "gqa": W.GQA_CAUSAL, "long": W.LONG_D64, "peak": W.PEAK}
# The attention kernel's sources and the committed counter summary of each
# path (INT8/FP8 and FP4): a summary counts only while its hash matches.
KERNEL_SOURCES = {
    "int8": ["quantized_attention_channel_amd/csrc/attn_kernel.hip",
             "quantized_attention_channel_amd/csrc/attn_schedule.h",
             "quantized_attention_channel_amd/csrc/sage_device.h"],
    "fp4": ["quantized_attention_channel_amd/csrc/fp4_kernels.hip",
            "quantized_attention_channel_amd/csrc/attn_schedule.h",
            "quantized_attention_channel_amd/csrc/sage_device.h"],
}
COUNTERS_MD = {"int8": os.path.join(ROOT, "profiles", "attn_fwd_peak_counters.md"),
               "fp4": os.path.join(ROOT, "profiles", "attn_fp4_peak_counters.md")}


def kernel_source_hash(path: str = "int8") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_ops(w: W.Workload) -> float:
    return w.attention_ops()


class Plan:
    """Preallocated buffers and the three C-ABI calls of one step."""

    def __init__(self, w: W.Workload, pv: str, q, k, v, qk_gran: str = "per_block"):
        import quantized_attention_channel_amd as sage
        self.sage, self.w, self.pv = sage, w, pv
        self.shape = sage.shape_of(q, k, w.layout, qk_gran)
        s = self.shape
        blk_q, blk_k, _ = sage.sage_block_sizes(w.d, qk_gran)
        dev = q.device
        npad = sage.sage_v_codes_stride(w.N)
        self.q, self.k, self.v = q, k, v
        self.o = torch.empty_like(q)
        self.q8 = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.int8, device=dev)
        self.sq = torch.empty((w.B, w.Hq, -(-w.N // blk_q)), dtype=torch.float32, device=dev)
        self.k8 = torch.empty((w.B, w.Hkv, w.N, w.d), dtype=torch.int8, device=dev)
        self.sk = torch.empty((w.B, w.Hkv, -(-w.N // blk_k)), dtype=torch.float32, device=dev)
        self.mu = torch.empty((w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
        if pv == "fp8":
            self.vp = torch.empty((w.B, w.Hkv, w.d, npad), dtype=torch.uint8, device=dev)
            self.sv = torch.empty((w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
        else:
            self.vp = torch.empty((w.B, w.Hkv, w.d, npad), dtype=q.dtype, device=dev)
            self.sv = None
        lib = sage.lib
        nws = max(lib.sage_quant_qk_workspace_bytes(ctypes.byref(s)), lib.sage_quant_v_workspace_bytes(ctypes.byref(s)))
        self.ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
        self.full_ws = torch.empty(max(sage.sage_workspace_bytes(s, pv), 256), dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        P = sage._ptr
        self.args_qk = (ctypes.byref(s), P(q), P(k), P(self.q8), P(self.sq), P(self.k8), P(self.sk), P(self.mu),
                        P(self.ws), self.ws.numel(), self.stream)
        self.args_v = (ctypes.byref(s), P(v), P(self.vp), P(self.sv), P(self.ws), self.ws.numel(), self.stream)
        self.args_vt = (ctypes.byref(s), P(v), P(self.vp), self.stream)
        self.args_attn = (ctypes.byref(s), P(self.q8), P(self.sq), P(self.k8), P(self.sk), P(self.vp), P(self.sv),
                          P(self.o), int(w.causal), float(w.sm_scale), sage.PV_DTYPES[pv], self.stream)
        self.args_full = (ctypes.byref(s), P(q), P(k), P(v), P(self.o), int(w.causal), float(w.sm_scale),
                          sage.PV_DTYPES[pv], P(self.full_ws), self.full_ws.numel(), self.stream)

    def quant(self):
        lib, chk = self.sage.lib, self.sage._check
        chk(lib.sage_quant_qk(*self.args_qk), "sage_quant_qk")
        if self.pv == "fp8":
            chk(lib.sage_quant_v(*self.args_v), "sage_quant_v")
        else:
            chk(lib.sage_transpose_v(*self.args_vt), "sage_transpose_v")

    def attention(self):
        self.sage._check(self.sage.lib.sage_attn_fwd_codes(*self.args_attn), "sage_attn_fwd_codes")

    def fused_entry(self):
        self.sage._check(self.sage.lib.sage_attn_fwd(*self.args_full), "sage_attn_fwd")


class Fp4Plan:
    """The FP4 microscaling variant: sage_quant_fp4 + sage_attn_fwd_fp4_codes
    per step (the kernels sage_attn_fwd_fp4 enqueues)."""

    def __init__(self, w: W.Workload, q, k, v):
        import quantized_attention_channel_amd as sage
        self.sage, self.w, self.pv = sage, w, "fp4"
        self.shape = s = sage.shape_of(q, k, w.layout)
        dev = q.device
        self.o = torch.empty_like(q)
        self.codes = c = sage.fp4_buffers(s, dev)
        lib = sage.lib
        self.ws = torch.empty(max(lib.sage_quant_fp4_workspace_bytes(ctypes.byref(s)), 256), dtype=torch.uint8,
                              device=dev)
        self.full_ws = torch.empty(max(sage.sage_fp4_workspace_bytes(s), 256), dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        P = sage._ptr
        self.args_quant = (ctypes.byref(s), P(q), P(k), P(v), float(w.sm_scale), P(c["q_codes"]), P(c["q_scale"]),
                           P(c["k_codes"]),
                           P(c["k_scale"]), P(c["k_mean"]), P(c["v_codes"]), P(c["v_scale"]), P(self.ws),
                           self.ws.numel(), self.stream)
        self.args_attn = (ctypes.byref(s), P(c["q_codes"]), P(c["q_scale"]), P(c["k_codes"]), P(c["k_scale"]),
                          P(c["v_codes"]), P(c["v_scale"]), P(self.o), int(w.causal), self.stream)
        self.args_full = (ctypes.byref(s), P(q), P(k), P(v), P(self.o), int(w.causal), float(w.sm_scale),
                          P(self.full_ws), self.full_ws.numel(), self.stream)

    def quant(self):
        self.sage._check(self.sage.lib.sage_quant_fp4(*self.args_quant), "sage_quant_fp4")

    def attention(self):
        self.sage._check(self.sage.lib.sage_attn_fwd_fp4_codes(*self.args_attn), "sage_attn_fwd_fp4_codes")

    def fused_entry(self):
        self.sage._check(self.sage.lib.sage_attn_fwd_fp4(*self.args_full), "sage_attn_fwd_fp4")


def time_steps(plan: Plan, steps: int, warmup: int):
    for _ in range(warmup):
        plan.quant()
        plan.attention()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        plan.quant()
        e1.record()
        plan.attention()
        e2.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    quant = [a.elapsed_time(b) for a, b, _ in ev]
    attn = [b.elapsed_time(c) for _, b, c in ev]
    gpu_ms = sum(a.elapsed_time(c) for a, _, c in ev) / steps
    return wall * 1e3, gpu_ms, sum(quant) / steps, sum(attn) / steps, statistics.median(quant), statistics.median(attn)


def time_fused_entry(plan: Plan, steps: int):
    plan.fused_entry()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.fused_entry()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def counters_traffic(w: W.Workload, pv: str, qk_gran: str):
    """HBM bytes per attention launch and the vector/matrix utilisation from the
    committed rocprofv3 counter summary, or (None, None) when it is missing,
    the kernel sources changed since, or it was taken on another configuration."""
    path = "fp4" if pv == "fp4" else "int8"
    md = COUNTERS_MD[path]
    if not os.path.exists(md):
        return None, None
    text = open(md).read()
    def grab(key):
        m = re.search(rf"^{key}:\s*([0-9A-Za-z_.+-]+)\s*$", text, flags=re.M)
        return m.group(1) if m else None
    same_config = (grab("counters_workload") == w.name and grab("counters_causal") == str(int(w.causal))
                   and grab("counters_pv") == pv and grab("counters_qk_gran") == qk_gran)
    vals = [grab(k) for k in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "copy_fetch_factor",
                              "copy_write_factor")]
    if grab("kernel_source_sha256") != kernel_source_hash(path) or not same_config or any(v is None for v in vals):
        return None, None
    fetch, write, ff, fw = (float(v) for v in vals)
    util = {k: float(grab(k)) for k in ("valu_busy_pct", "mfma_util_pct") if grab(k) is not None}
    return (fetch * ff + write * fw) * 1024.0, util or None


def cpu_baseline(w: W.Workload, pv: str, rows: int, qk_gran: str = "per_block"):
    """The oracle, as it stands, on a bounded sample: batch 0 / head 0 of the
    workload, its Q/K/V quantisation in full and `rows` query rows of attention."""
    import numpy as np
    from oracle import sage_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    one = w.with_(B=1, Hq=1, Hkv=1)
    q, k, v = W.generate(one)
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    sel = np.linspace(0, w.N - 1, rows).round().astype(np.int64)
    t0 = time.perf_counter()
    blk = ((sage_ref.PER_THREAD_BLK_Q, sage_ref.PER_THREAD_BLK_K) if qk_gran == "per_thread"
           else (sage_ref.BLK_Q, sage_ref.BLK_K))
    if pv == "fp4":
        sage_ref.sage_attention_fp4(qn, kn, vn, dtype=w.dtype, is_causal=w.causal, sm_scale=w.sm_scale,
                                    layout=w.layout, rows=np.unique(sel))
    else:
        sage_ref.sage_attention(qn, kn, vn, dtype=w.dtype, is_causal=w.causal, sm_scale=w.sm_scale, pv=pv,
                                layout=w.layout, rows=np.unique(sel), blk_q=blk[0], blk_k=blk[1])
    dt = time.perf_counter() - t0
    if w.causal:
        ops = float(sum(4.0 * (int(i) + 1) * w.d for i in np.unique(sel)))
    else:
        ops = 4.0 * len(np.unique(sel)) * w.N * w.d
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": (f"batch 0, head 0 of {w.B * w.Hq}: Q/K/V quantisation of that head in full "
                       f"(N={w.N}) plus {len(np.unique(sel))} of {w.N} query rows of attention; "
                       f"TOPS counted as 4*rows*N*d{' (causal: visible keys only)' if w.causal else ''}")}


def cpu_configs(rows_sample: int = 512):
    """The oracle on the host cores for every workload (one JSON line each).

    The tiny and the outlier workload run in full. The GQA causal, d = 64 and
    peak workloads run their quantisation in full and attention for
    `rows_sample` query rows of every (batch, head) plus the edge rows; their
    whole-workload time is an extrapolation, t_quant + t_rows * (all visible
    pairs / sampled visible pairs), and is labelled as such."""
    import numpy as np
    from oracle import sage_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    for w in (W.TINY, W.MID_OUTLIER, W.GQA_CAUSAL, W.LONG_D64, W.PEAK):
        full = w in (W.TINY, W.MID_OUTLIER)
        q, k, v = W.generate(w)
        qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), w.layout) for t in (q, k, v))
        t0 = time.perf_counter()
        parts = sage_ref.quant_qk(qn, kn)
        if w.pv == "fp8":
            parts["v8"], parts["v_scale"] = sage_ref.quant_v_fp8(vn)
        t_quant = time.perf_counter() - t0
        if full:
            rows = np.arange(w.N)
        else:
            rows = np.unique(np.concatenate([np.linspace(0, w.N - 1, rows_sample).round().astype(np.int64),
                                             [0, 1, w.N - 2, w.N - 1]]))
        G = w.Hq // w.Hkv
        t1 = time.perf_counter()
        for b in range(w.B):
            for h in range(w.Hq):
                g = h // G
                sub = {"q8": parts["q8"][b:b + 1, h:h + 1], "q_scale": parts["q_scale"][b:b + 1, h:h + 1],
                       "k8": parts["k8"][b:b + 1, g:g + 1], "k_scale": parts["k_scale"][b:b + 1, g:g + 1]}
                if w.pv == "fp8":
                    sub["v8"], sub["v_scale"] = parts["v8"][b:b + 1, g:g + 1], parts["v_scale"][b:b + 1, g:g + 1]
                sage_ref.sage_attention(qn[b:b + 1, h:h + 1], kn[b:b + 1, g:g + 1], vn[b:b + 1, g:g + 1],
                                        dtype=w.dtype, is_causal=w.causal, sm_scale=w.sm_scale, pv=w.pv, rows=rows,
                                        parts=sub)
            print(f"  oracle {w.name}: batch {b} done ({time.perf_counter() - t1:.0f} s)", file=sys.stderr, flush=True)
        t_rows = time.perf_counter() - t1
        pairs = lambda r: float((r + 1).sum()) if w.causal else float(len(r)) * w.N   # visible (query, key) pairs
        frac = pairs(rows) / pairs(np.arange(w.N))
        t_total = t_quant + t_rows / frac
        rec = {"workload": w.name, "pv": w.pv, "causal": w.causal, "cores": int(threads),
               "quant_s": round(t_quant, 2), "attention_rows": int(len(rows)), "attention_s": round(t_rows, 2),
               "kind": "measured in full" if full else "extrapolated: quant in full + sampled rows scaled by visible pairs",
               "seconds_whole_workload": round(t_total, 1),
               "TOPS": w.attention_ops() / t_total / 1e12}
        print(json.dumps(rec), flush=True)


def copy_calibration():
    """A plain device copy of known size, for scaling HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def copy_bandwidth() -> float:
    """Measured device copy rate in GB/s (bytes read plus bytes written per
    second) over a 1 GiB buffer: the practical ceiling for the HBM-bound
    quantisation kernels."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    del src, dst
    return 2.0 * n / (ms * 1e-3) / 1e9


def host_info():
    """CPU model and the BLAS behind NumPy, for the CPU baseline record."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "numpy_blas": blas}


def measure(w: W.Workload, pv: str, steps: int, warmup: int, qk_gran: str = "per_block"):
    q, k, v = W.generate(w, device="cuda")
    plan = Fp4Plan(w, q, k, v) if pv == "fp4" else Plan(w, pv, q, k, v, qk_gran)
    wall_ms, gpu_ms, quant_ms, attn_ms, quant_med, attn_med = time_steps(plan, steps, warmup)
    fused_ms = time_fused_entry(plan, max(3, steps // 4))
    ops = counted_ops(w)
    return dict(wall_ms=wall_ms, gpu_ms=gpu_ms, quant_ms=quant_ms, attn_ms=attn_ms, fused_ms=fused_ms,
                quant_median_ms=quant_med, attn_median_ms=attn_med,
                tops=ops / (wall_ms * 1e-3) / 1e12, attn_tops=ops / (attn_ms * 1e-3) / 1e12,
                quant_bytes=3.0 * (w.B * w.Hq * w.N * w.d + 2 * w.B * w.Hkv * w.N * w.d))


def measure_varlen(w: W.VarlenWorkload, steps: int, warmup: int):
    """One sage_attn_fwd_varlen (or, pv "fp4", sage_attn_fwd_fp4_varlen) call
    per step (quantisation and attention of every sequence of the packed
    batch), timed with HIP events."""
    import quantized_attention_channel_amd as sage
    q, k, v, cq, ck = W.generate_varlen(w, device="cuda")
    mq, mk = max(w.lens_q), max(w.lens_k)
    shape = sage.varlen_shape_of(q, k, cq, mq, mk)
    need = sage.sage_fp4_varlen_workspace_bytes(shape) if w.pv == "fp4" else \
        sage.sage_varlen_workspace_bytes(shape, w.pv)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)

    def run():
        if w.pv == "fp4":
            sage.sage_attn_fwd_fp4_varlen(q, k, v, cq, ck, mq, mk, is_causal=w.causal, sm_scale=w.sm_scale,
                                          out=o, workspace=ws)
        else:
            sage.sage_attn_fwd_varlen(q, k, v, cq, ck, mq, mk, is_causal=w.causal, sm_scale=w.sm_scale,
                                      pv_dtype=w.pv, out=o, workspace=ws)
    for _ in range(warmup):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    ops = w.attention_ops()
    return {"value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "workload": w.name, "sequences": w.B, "tokens": sum(w.lens_q), "causal": w.causal, "pv": w.pv,
            "ops_per_step": ops}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="peak", help="peak|tiny|mid|gqa|long or a full workload name")
    ap.add_argument("--pv", default=None, help="fp8|fp16|fp4 (default: the workload's; fp4 = the FP4 "
                    "microscaling variant, MXFP4 Q/K/P/V)")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's causal flag")
    ap.add_argument("--qk-gran", default="per_block", choices=["per_block", "per_thread"],
                    help="granularity of the Q/K INT8 scales")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the causal and per-thread variants of the peak workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--copy-calibration", action="store_true", help="run only a 1 GiB device copy")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="time only the CPU oracle on every workload (no GPU; several minutes)")
    args = ap.parse_args()
    if args.cpu_configs:
        cpu_configs()
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantised attention "
              "path here is a single-GPU kernel; see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    w = ALIASES.get(args.workload) or W.ALL[args.workload]
    if args.causal is not None:
        w = w.with_(causal=bool(args.causal))
    pv = args.pv or w.pv

    if pv == "fp4" and args.qk_gran != "per_block":
        print("the FP4 variant has fixed MX blocks: --qk-gran must be per_block", file=sys.stderr)
        sys.exit(2)
    r = measure(w, pv, args.steps, args.warmup, args.qk_gran)
    copy_gbps = copy_bandwidth()
    traffic, util = counters_traffic(w, pv, args.qk_gran)
    peak = PEAK_FP4_TOPS if pv == "fp4" else PEAK_TOPS
    roof = {"bound": "mfma", "achieved": round(r["attn_tops"], 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(r["attn_tops"] / peak, 4), "traffic": traffic,
            "kernel": ("attn_fp4_kernel" if pv == "fp4" else
                       "attn_fwd_fine_kernel" if args.qk_gran == "per_thread" else "attn_fwd_kernel"),
            "ops_per_launch": counted_ops(w),
            "mean_launch_ms": round(r["attn_ms"], 4), "median_launch_ms": round(r["attn_median_ms"], 4)}
    if util:
        roof["counters_pct"] = util     # rocprofv3 VALUBusy / MfmaUtil of the same kernel (profiles/)
    out = {
        "metric": METRIC, "value": round(r["tops"], 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["wall_ms"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "int8+fp8_e4m3", "fp4": "mxfp4_e2m1"}.get(pv, f"int8+{w.dtype}"),
        "data": "synthetic: seeded normal Q/K/V, per-channel K offsets (workloads.py)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "pv": pv, "layout": w.layout, "input_dtype": w.dtype,
                   "qk_gran": args.qk_gran},
        "mfma_peak_frac": round(r["tops"] / peak, 4),
        "roofline": roof,
        "breakdown_ms": {"gpu_step": round(r["gpu_ms"], 4), "quant": round(r["quant_ms"], 4),
                         "attention": round(r["attn_ms"], 4), "sage_attn_fwd_single_call": round(r["fused_ms"], 4),
                         "quant_median": round(r["quant_median_ms"], 4), "attention_median": round(r["attn_median_ms"], 4)},
        "quant_hbm": {"algorithmic_bytes": r["quant_bytes"], "copy_GBps": round(copy_gbps, 1),
                      "frac_of_copy": round(r["quant_bytes"] / (r["quant_ms"] * 1e-3) / 1e9 / copy_gbps, 4),
                      "GBps": round(r["quant_bytes"] / (r["quant_ms"] * 1e-3) / 1e9, 1),
                      "frac_of_8TBps": round(r["quant_bytes"] / (r["quant_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    if w is W.PEAK and args.qk_gran == "per_block" and pv != "fp4" and not args.no_variants:
        def variant(rv, pk=PEAK_TOPS):
            return {"value": round(rv["tops"], 2), "ms_per_step": round(rv["wall_ms"], 4),
                    "attention_tops": round(rv["attn_tops"], 2),
                    "attention_frac": round(rv["attn_tops"] / pk, 4),
                    "attention_ms": round(rv["attn_ms"], 4), "quant_ms": round(rv["quant_ms"], 4)}
        out["variants"] = {"causal": variant(measure(w.with_(causal=True), pv, args.steps, args.warmup)),
                           "per_thread": variant(measure(w, pv, args.steps, args.warmup, "per_thread")),
                           "varlen": measure_varlen(W.VARLEN_PREFILL, args.steps, args.warmup),
                           # the FP4 microscaling variant: attention_frac against the 10.1 PFLOP/s FP4 peak
                           "fp4": variant(measure(w, "fp4", args.steps, args.warmup), PEAK_FP4_TOPS),
                           "fp4_causal": variant(measure(w.with_(causal=True), "fp4", args.steps, args.warmup),
                                                 PEAK_FP4_TOPS),
                           "fp4_varlen": measure_varlen(W.VARLEN_PREFILL.with_(pv="fp4"), args.steps,
                                                        args.warmup)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, pv, args.cpu_rows, args.qk_gran)
        out["cpu_baseline"].update(host_info())
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
