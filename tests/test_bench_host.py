"""Host checks of the benchmark's bookkeeping (CPU only).

The committed counter summary is attached to a benchmark line only for the
configuration and the kernel sources it was taken on.
"""
import bench
import workloads as W


def test_counters_attach_only_to_their_own_configuration():
    import os
    import re
    for path, pv in (("int8", "fp8"), ("fp4", "fp4")):
        if not os.path.exists(bench.COUNTERS_MD[path]):
            assert bench.counters_traffic(W.PEAK, pv, "per_block") == (None, None)
            continue
        text = open(bench.COUNTERS_MD[path]).read()
        recorded = re.search(r"^kernel_source_sha256:\s*(\S+)", text, flags=re.M).group(1)
        traffic, util = bench.counters_traffic(W.PEAK, pv, "per_block")
        if recorded == bench.kernel_source_hash(path):
            assert traffic is not None and traffic > 0
            assert set(util) == {"valu_busy_pct", "mfma_util_pct"} and all(0 < v <= 100 for v in util.values())
        else:                                              # sources changed since: no stale counters
            assert (traffic, util) == (None, None)
    for w, pv, gran in [(W.PEAK.with_(causal=True), "fp8", "per_block"), (W.PEAK, "fp16", "per_block"),
                        (W.PEAK, "fp8", "per_thread"), (W.MID_OUTLIER, "fp8", "per_block"),
                        (W.PEAK.with_(causal=True), "fp4", "per_block")]:
        assert bench.counters_traffic(w, pv, gran) == (None, None)


def test_counted_ops_follow_the_metric():
    # 4*B*H*N^2*d, halved for causal
    assert bench.counted_ops(W.PEAK) == 4.0 * 1 * 32 * 32768 ** 2 * 128
    assert bench.counted_ops(W.PEAK.with_(causal=True)) == 2.0 * 32 * 32768 ** 2 * 128


def test_more_than_one_gpu_exits_with_a_message():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
