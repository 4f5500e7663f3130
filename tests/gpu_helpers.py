"""Helpers for the GPU parity tests: move seeded workloads to the device, run the library's hot
path through its C ABI, and compare with the oracle (no attention arithmetic here)."""
import sys

import numpy as np
import torch

import attention_paged_kv_amd as pa
from attention_paged_kv_amd import workloads as W

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f32": 1e-5}          # max-abs contract for outputs
ROW_REL_L2 = {"bf16": 1e-2, "f32": 1e-5}   # stricter per-row relative L2 gate


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "i8":
        return torch.from_numpy(a.astype(np.int8, copy=False)).to(DEV)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host_array(t, dtype):
    if dtype == "i8":
        return t.cpu().numpy()
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def int_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class GpuState:
    """Device caches for one workload, advanced step by step like the host oracle's copies."""

    def __init__(self, w, kc=None, vc=None):
        self.w = w
        self.kc = dev_tensor(w.k_cache0 if kc is None else kc, w.cache_dtype)
        self.vc = dev_tensor(w.v_cache0 if vc is None else vc, w.cache_dtype)
        self.ks = self.vs = None
        if w.cache_dtype == "i8":
            self.ks = torch.from_numpy(np.ascontiguousarray(w.k_scale)).to(DEV)
            self.vs = torch.from_numpy(np.ascontiguousarray(w.v_scale)).to(DEV)

    def inputs(self, st):
        return dict(q=dev_tensor(st.q, self.w.dtype), k=dev_tensor(st.k_new, self.w.dtype),
                    v=dev_tensor(st.v_new, self.w.dtype), slots=int_tensor(st.slot_mapping),
                    bt=int_tensor(st.block_tables), sl=int_tensor(st.seq_lens), qsl=int_tensor(st.query_start_loc))

    def step(self, st, append=True, window=0, max_q_len=0):
        x = self.inputs(st)
        if append:
            pa.append_kv(x["k"], x["v"], x["slots"], self.kc, self.vc, self.ks, self.vs)
        out = torch.empty_like(x["q"])
        pa.attention(x["q"], self.kc, self.vc, x["bt"], x["sl"], x["qsl"], self.w.scale, out, window=window,
                     k_scale=self.ks, v_scale=self.vs, max_q_len=max_q_len)
        torch.cuda.synchronize()
        return host_array(out, self.w.dtype)


def compare(out_gpu, out_ref, dtype, rows=None, what=""):
    g = W.to_float(out_gpu, dtype).astype(np.float64)
    r = W.to_float(out_ref, dtype).astype(np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    maxabs = float(err.max()) if err.size else 0.0
    num = np.sqrt(((g - r) ** 2).sum(axis=-1))
    den = np.sqrt((r ** 2).sum(axis=-1)) + 1e-30
    rel = float((num / den).max()) if num.size else 0.0
    say(f"  {what}: max-abs {maxabs:.3e} (tol {TOL[dtype]:.0e}), max row rel-L2 {rel:.3e}")
    assert maxabs <= TOL[dtype], f"{what}: max-abs {maxabs} > {TOL[dtype]}"
    assert rel <= ROW_REL_L2[dtype], f"{what}: row rel-L2 {rel} > {ROW_REL_L2[dtype]}"
    return maxabs, rel


def tile_rows(q0, q_len, pos_per_tile, rng, n_random=16, waves=8):
    """Query rows that touch every prefill tile of one request: each tile's first and last row,
    one row in each wave's slice of the tile (a wave holds pos_per_tile / waves consecutive
    positions), plus random rows.  Rows are token indices (q0 + local row)."""
    rows = set()
    per_wave = max(1, pos_per_tile // waves)
    n_tiles = (q_len + pos_per_tile - 1) // pos_per_tile
    for i in range(n_tiles):
        lo, hi = i * pos_per_tile, min(q_len, (i + 1) * pos_per_tile)
        rows.update((lo, hi - 1))
        for wv in range(waves):
            r = lo + wv * per_wave + (3 * i + 5 * wv) % per_wave
            if r < hi:
                rows.add(r)
    rows.update(int(x) for x in rng.integers(0, q_len, n_random))
    return q0 + np.array(sorted(rows), dtype=np.int64)
