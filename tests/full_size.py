"""Full-size GPU parity shared by the per-block and per-thread tests.

The HIP path runs each workload at its full size, in the configuration the
benchmark times. Then:
* the integer stages (K mean, Q/K codes and scales; V codes and scales in FP8
  mode) are compared in full, bit for bit;
* the float output is compared with the oracle on one row of every 256-query
  work-group of every head (alternating between the work-group's two 128-query
  groups) plus the edge rows, head by head (cosine >= 0.9999, relative L1 <=
  1e-3) and pooled; against fp64 exact attention the pooled cosine must reach
  the method's bound;
* where asked, the oracle is also run under rejected readings of the method,
  and the HIP path must sit at most a quarter of each one's distance from the
  chosen reading, so the bounds tell the readings apart.
"""
import numpy as np
import torch

import workloads as W
from oracle import exact, sage_ref
from tests.parity_util import (COS_ORACLE, RL1_ORACLE, check_heads, cos, exact_rows_per_head,
                               oracle_rows_per_head, rel_l1, rows_per_head, say)


def _pooled(xs):
    return np.concatenate([np.ravel(x) for x in xs])


def run_full_size(sage, w, pv, gran, *, exact_bound, rejected_readings=()):
    blk_q, blk_k = ((sage_ref.PER_THREAD_BLK_Q, sage_ref.PER_THREAD_BLK_K) if gran == "per_thread"
                    else (sage_ref.BLK_Q, sage_ref.BLK_K))
    say("full workload", w.name, pv, gran, "causal" if w.causal else "")
    q, k, v = W.generate(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o = sage.sage_attn_fwd(qg, kg, vg, is_causal=w.causal, sm_scale=w.sm_scale, pv_dtype=pv,
                           tensor_layout=w.layout, qk_gran=gran)
    quant = sage.sage_quant_qk(qg, kg, tensor_layout=w.layout, qk_gran=gran)
    vq = sage.sage_quant_v(vg, tensor_layout=w.layout) if pv == "fp8" else None
    torch.cuda.synchronize()
    del qg, kg, vg
    qn, kn, vn = (sage_ref.as_hnd(t.float().numpy(), w.layout) for t in (q, k, v))
    parts = sage_ref.quant_qk(qn, kn, blk_q=blk_q, blk_k=blk_k)
    # integer stages in full
    assert np.array_equal(quant["k_mean"].cpu().numpy(), parts["k_mean"])
    assert np.array_equal(quant["q_scale"].cpu().numpy(), parts["q_scale"])
    assert np.array_equal(quant["k_scale"].cpu().numpy(), parts["k_scale"])
    assert np.array_equal(quant["q_codes"].cpu().numpy(), parts["q8"])
    assert np.array_equal(quant["k_codes"].cpu().numpy(), parts["k8"])
    if pv == "fp8":
        parts["v8"], parts["v_scale"] = sage_ref.quant_v_fp8(vn)
        assert np.array_equal(vq[1].cpu().numpy(), parts["v_scale"])
        assert np.array_equal(vq[0].cpu().numpy()[..., :w.N], parts["v8"])
    # float output, one row per work-group and head
    rows = rows_per_head(w.N, w.B * w.Hq)
    o_all = sage_ref.as_hnd(o.float().cpu().numpy(), w.layout)
    got = [o_all[i // w.Hq, i % w.Hq, r] for i, r in enumerate(rows)]
    kw = dict(dtype=w.dtype, causal=w.causal, sm_scale=w.sm_scale, pv=pv, rows=rows, blk_q=blk_q, blk_k=blk_k)
    ref = oracle_rows_per_head(sage_ref, qn, kn, vn, parts, **kw)
    ex = exact_rows_per_head(exact, qn, kn, vn, causal=w.causal, sm_scale=w.sm_scale, rows=rows)
    assert all(np.isfinite(g).all() for g in got)
    wc, wr = check_heads(got, ref)
    G, R, E = _pooled(got), _pooled(ref), _pooled(ex)
    c, r, ce = cos(G, R), rel_l1(G, R), cos(G, E)
    say(f"   {sum(len(x) for x in rows)} rows: cos={c:.7f} rel_l1={r:.2e} worst head cos={wc:.7f} "
        f"rel_l1={wr:.2e}; cos_exact={ce:.6f}")
    assert c >= COS_ORACLE and r <= RL1_ORACLE
    assert ce >= exact_bound
    for rej in rejected_readings:
        alt = _pooled(oracle_rows_per_head(sage_ref, qn, kn, vn, parts, rejected=rej, **kw))
        d_alt = rel_l1(alt, R)
        say(f"   rejected reading {rej}: {d_alt:.2e} from the oracle; HIP path {r:.2e}")
        assert r <= 0.25 * d_alt, f"the parity bound cannot tell {rej} from the method"
