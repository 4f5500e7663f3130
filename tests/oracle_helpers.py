"""Helpers shared by the CPU oracle tests (no attention arithmetic here)."""
import numpy as np

from attention_paged_kv_amd import workloads as W
import oracle


def oracle_step(w, step=None, rows=None, want_f64=True, caches=None, window=0):
    """Run one step through the oracle on copies of the workload's caches."""
    step = step if step is not None else w.steps[0]
    kc = (caches[0] if caches else w.k_cache0).copy()
    vc = (caches[1] if caches else w.v_cache0).copy()
    out, out64 = oracle.run_step(w, step, kc, vc, rows=rows, want_f64=want_f64, window=window)
    return out, out64, kc, vc


def logical_kv(w, step, kc, vc, b):
    """Read request b's keys/values back through its block table (for building dense inputs)."""
    s = int(step.seq_lens[b])
    pos = np.arange(s)
    slots = W.slots_for(step.block_tables, b, pos)
    NB = kc.shape[0]
    k2 = kc.reshape(NB * 16, w.num_kv_heads, w.head_dim)[slots]
    v2 = vc.reshape(NB * 16, w.num_kv_heads, w.head_dim)[slots]
    return W.to_float(k2, w.dtype).astype(np.float64), W.to_float(v2, w.dtype).astype(np.float64)
