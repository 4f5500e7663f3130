#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: append this step's K/V into the paged cache,
then causal attention of every query row (decode splits + merge, and prefill/chunk tiles where
the batch has them).  Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c3|c4|c5|c1] [--window N]
                    [--kv bf16|i8] [--verify K] [--chunks N] [--no-cpu-baseline] [--only]

Prints one JSON line.  The default workload is the 32-request bf16 decode batch (32/32 heads,
d=128, contexts U[512, 4096], 16384-block pool); its metric is KV-read GB/s.  The default run also
times, in the same process, the 8k causal prefill (c3), the mixed chunked step (c4) and the
length-skewed long decode (c5), each under "workloads" with its own roofline object; prefill
workloads warm up for at least 60 steps (compute-bound launches speed up over a run's first few
dozen).  --only times the named workload alone.  --window N runs the
same workload with a sliding window of N keys per query row; work counts then cover only the keys
and pairs inside the windows.  --kv i8 keeps the workload's shapes and lengths over an 8-bit cache
(int8 codes, fp32 scale per KV head and channel; c2 .. c5): KV bytes count 1 byte per
element.  --verify K turns a decode workload into a verification step: each request appends and
attends its last K tokens (same lengths and tables), still one read of every visible key.
--chunks N (c3) appends and attends the prompt as N equal chunks, each over the keys cached before
it; a step is then the whole prompt, and the default run reports four 2048-token chunks next to
the one-shot prefill ("c3_chunks4", with chunked_over_one_shot = the ratio of their GPU times).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn throughput: decode KV-read GB/s, prefill TFLOPS, % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_VEC_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources a kernel's HBM traffic depends on: the kernel, its helpers and the host code that sets its
# launch (split lengths, workgroup forms, tile sizes).
KERNEL_SOURCES = {
    "decode_split": ["attention_paged_kv_amd/csrc/pa_decode.hip", "attention_paged_kv_amd/csrc/pa_decode_i8.hip",
                     "attention_paged_kv_amd/csrc/pa_rows.h", "attention_paged_kv_amd/csrc/pa_common.h",
                     "attention_paged_kv_amd/csrc/pa_internal.h", "attention_paged_kv_amd/csrc/pa_api.hip"],
    "prefill_tile": ["attention_paged_kv_amd/csrc/pa_prefill.hip", "attention_paged_kv_amd/csrc/pa_common.h",
                     "attention_paged_kv_amd/csrc/pa_internal.h", "attention_paged_kv_amd/csrc/pa_api.hip"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary
    (profiles/hbm_traffic.txt), or None if absent or taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    m = hashlib.sha256()
    for fn in KERNEL_SOURCES[kernel]:
        m.update(open(os.path.join(ROOT, fn), "rb").read())
    src = m.hexdigest()[:16]
    for line in open(path):
        f = line.split()
        if len(f) == 8 and not line.startswith("#") and f[0] == kernel and f[1] == workload and f[7] == src:
            return int(f[6])
    return None


def cpu_baseline(w, steps, is_decode, kv_bytes, window=0):
    """Time the fp64 CPU oracle on the host cores over a bounded sample of the same workload.

    Decode workloads (and the tiny fp32 sequence) run whole steps, repeated until ~10 s; prefill
    workloads run a strided sample of query rows (all decode rows of a mixed batch are kept), and
    the rate is the algorithmic FLOPs of the sampled rows over the oracle's time."""
    import oracle
    from attention_paged_kv_amd import accounting as A
    threads = oracle.default_threads()
    kcs, vcs = w.k_cache0.copy(), w.v_cache0.copy()
    if is_decode or w.dtype == "f32":
        reps, t_cpu = 0, 0.0
        while t_cpu < 10.0 and reps < 50:
            for st in steps:
                ta = time.perf_counter()
                oracle.run_step(w, st, kcs, vcs, num_threads=threads, window=window)
                t_cpu += time.perf_counter() - ta
            reps += 1
        per = t_cpu / reps
        if is_decode:
            val, unit = kv_bytes / per / 1e9, "GB/s"
        else:
            fl = sum(A.attention_flops(st.q_lens, st.seq_lens, w.num_q_heads, w.head_dim, window) for st in steps)
            val, unit = fl / per / 1e12, "TFLOP/s"
        sample = f"whole {w.name} step (append + attention of every row), {reps} run(s), {per:.3f} s per step"
    else:
        st = steps[0]
        ql = st.q_lens
        rows, pos = [], []
        for b in range(st.num_seqs):
            q0, n = int(st.query_start_loc[b]), int(ql[b])
            ctx = int(st.seq_lens[b]) - n
            stride = 1 if n == 1 else 64
            for r in range(0, n, stride):
                rows.append(q0 + r)
                pos.append(ctx + r)
        rows = np.array(rows, np.int32)
        seen = np.array(pos, np.int64) + 1
        if window > 0:
            seen = np.minimum(seen, window)
        fl = 4 * w.head_dim * w.num_q_heads * int(np.sum(seen))
        oracle.append(st.k_new, st.v_new, st.slot_mapping, kcs, vcs)
        ta = time.perf_counter()
        oracle.attention(st.q, kcs, vcs, st.block_tables, st.seq_lens, st.query_start_loc, w.scale, rows=rows,
                         num_threads=threads, window=window)
        per = time.perf_counter() - ta
        val, unit = fl / per / 1e12, "TFLOP/s"
        sample = (f"{len(rows)} of {st.num_tokens} query rows of {w.name} (every 64th prefill row, every decode "
                  f"row), all heads, {per:.2f} s")
    return {"value": round(val, 6), "unit": unit, "cores": threads, "kind": "oracle", "sample": sample}


def host_cpu():
    """(logical CPUs of the host, CPU model) for the baseline's context."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count() or 0, model


def measure(cfg, kv, win, verify, steps_n, warmup, dev, want_cpu=False, chunks=1):
    """Times one workload (append + attention per step) and returns its JSON record.  chunks > 1
    (one-request prefill workloads): the prompt is appended and attended as that many equal chunks,
    each over the keys cached before it, and a "step" is the whole sequence of chunks."""
    import torch

    import attention_paged_kv_amd as pa
    from attention_paged_kv_amd import accounting as A
    from attention_paged_kv_amd import workloads as W

    t0 = time.time()
    w = W.CONFIGS[cfg](cache="i8") if kv == "i8" else W.CONFIGS[cfg]()
    if verify > 1:
        w = W.verify_variant(w, verify)
    if chunks > 1:
        S = int(w.steps[0].seq_lens[0])
        w = W.chunked_steps(w, [S // chunks] * (chunks - 1) + [S - (S // chunks) * (chunks - 1)])
    log(f"generated {w.name} in {time.time() - t0:.1f}s")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # c1 is a 17-step sequence; its "step" is the whole sequence.  Others are one step.
    steps = w.steps
    if w.cache_dtype == "i8":
        kc = torch.from_numpy(w.k_cache0).to(dev)
        vc = torch.from_numpy(w.v_cache0).to(dev)
        ks = torch.from_numpy(w.k_scale).to(dev)
        vs = torch.from_numpy(w.v_scale).to(dev)
    else:
        kc = to_dev(w.k_cache0)
        vc = to_dev(w.v_cache0)
        ks = vs = None
    dsteps = []
    for st in steps:
        dsteps.append(dict(q=to_dev(st.q), k=to_dev(st.k_new), v=to_dev(st.v_new),
                           slots=to_dev(st.slot_mapping.astype(np.int32)), bt=to_dev(st.block_tables),
                           sl=to_dev(st.seq_lens), qsl=to_dev(st.query_start_loc),
                           out=torch.empty(st.q.shape, dtype=tdt, device=dev),
                           max_q=int(st.q_lens.max())))     # a scheduler knows its step's longest q_len
    ws_need = max(pa.workspace_size(st.num_seqs, st.num_tokens, st.block_tables.shape[1], w.num_q_heads, kc, ks, vs)
                  for st in steps)
    ws = torch.zeros(max(ws_need, 256), dtype=torch.uint8, device=dev)

    def run_step():
        for d in dsteps:
            pa.append_kv(d["k"], d["v"], d["slots"], kc, vc, ks, vs)
            pa.attention(d["q"], kc, vc, d["bt"], d["sl"], d["qsl"], w.scale, d["out"], workspace=ws, window=win,
                         k_scale=ks, v_scale=vs, max_q_len=d["max_q"])

    # algorithmic work of one step
    kv_bytes = sum(A.kv_read_bytes(st.seq_lens, w.num_kv_heads, w.head_dim, w.esz, st.q_lens, win) for st in steps)
    flops = sum(A.attention_flops(st.q_lens, st.seq_lens, w.num_q_heads, w.head_dim, win) for st in steps)
    tile_flops = sum(A.attention_flops(st.q_lens[st.q_lens > 1], st.seq_lens[st.q_lens > 1], w.num_q_heads,
                                       w.head_dim, win) for st in steps)
    dec_bytes = sum(A.kv_read_bytes(st.seq_lens[st.q_lens == 1], w.num_kv_heads, w.head_dim, w.esz,
                                    st.q_lens[st.q_lens == 1], win) for st in steps)
    wname = w.name if win == 0 else f"{w.name}-w{win}"     # names the workload in the counter summary

    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps_n):
        run_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / steps_n

    # per-kernel durations from hipEvents the library records around its own launches (same stream)
    pa.timing_reset()
    pa.timing_enable(True)
    for _ in range(steps_n):
        run_step()
    torch.cuda.synchronize()
    kern = {}
    for name in ("append", "decode_split", "decode_merge", "prefill_tile"):
        ms, n = pa.timing_read(name)
        if n:
            kern[name] = {"avg_us": 1e3 * ms / n, "launches_per_step": n / steps_n}
    pa.timing_enable(False)
    pa.timing_reset()

    is_decode = cfg in ("c2", "c5")
    extra = {}
    if is_decode:
        unit = "GB/s"
        value = kv_bytes / (ms_per_step * 1e-3) / 1e9
        dk = kern["decode_split"]
        per_launch = kv_bytes / dk["launches_per_step"]
        achieved = per_launch / (dk["avg_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "decode_split", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode_split", wname),
                "algorithmic_bytes_per_launch": int(per_launch)}
    elif w.dtype == "f32":
        unit = "TFLOP/s"
        value = flops / (ms_per_step * 1e-3) / 1e12
        dk = kern["decode_split"]
        per_launch = flops / dk["launches_per_step"]
        achieved = per_launch / (dk["avg_us"] * 1e-6) / 1e12
        roof = {"bound": "alu", "kernel": "decode_split", "achieved": round(achieved, 4),
                "peak": FP32_VEC_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP32_VEC_PEAK_TFLOPS, 6),
                "traffic": None, "algorithmic_flops_per_launch": int(per_launch)}
    else:
        unit = "TFLOP/s"
        value = flops / (ms_per_step * 1e-3) / 1e12
        tk = kern["prefill_tile"]
        per_launch = tile_flops / tk["launches_per_step"]
        achieved = per_launch / (tk["avg_us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": "prefill_tile", "achieved": round(achieved, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("prefill_tile", wname),
                "algorithmic_flops_per_launch": int(per_launch)}
        if "decode_split" in kern and dec_bytes:
            # A mixed step runs its decode pass beside the tiles (on a side stream), so its events
            # also span the wait for compute units: time the decode rows as a batch of their own.
            dk = decode_rows_alone(pa, w, steps, dsteps, kc, vc, ks, vs, win, steps_n, dev)
            ach = dec_bytes / (dk["avg_us"] * 1e-6) / 1e9
            extra["decode_part"] = {"bound": "hbm", "kernel": "decode_split", "achieved": round(ach, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                    "avg_us": round(dk["avg_us"], 3), "merge_avg_us": round(dk["merge_us"], 3),
                                    "measured_as": "the step's decode rows as a batch of their own",
                                    "traffic": None, "algorithmic_bytes_per_launch": int(dec_bytes)}
            # the whole step against its own roofline: the longer of its compute and memory times
            t_roof = max(flops / (BF16_PEAK_TFLOPS * 1e12), kv_bytes / (HBM_PEAK_GBS * 1e9))
            extra["step_roofline_frac"] = round(t_roof / (gpu_ms / steps_n * 1e-3), 4)

    cpu = cpu_baseline(w, steps, is_decode, kv_bytes, win) if want_cpu else None
    rec = {
        "value": round(value, 2 if unit == "GB/s" else 3),
        "unit": unit,
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms / steps_n, 5),
        "steps": steps_n,
        "warmup": warmup,
        "dtype": w.dtype,
        "config": {"workload": wname, "description": w.description + (f", sliding window {win}" if win else ""),
                   "sliding_window": win, "kv_cache": w.cache_dtype, "num_seqs": int(steps[0].num_seqs),
                   "attention_calls_per_step": len(steps),
                   "q_tokens": int(sum(st.num_tokens for st in steps)),
                   "kv_read_bytes": int(kv_bytes), "flops": int(flops), "parallelism": "single-gpu"},
        "kernels": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in kern.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    rec.update(extra)
    del dsteps, kc, vc, ws
    torch.cuda.empty_cache()
    return rec


def decode_rows_alone(pa, w, steps, dsteps, kc, vc, ks, vs, win, steps_n, dev):
    """Average decode-split and merge durations of a one-step workload's q_len-1 rows attended as a
    batch of their own (same caches, tables and queries), from the library's per-launch events."""
    import torch
    st, d = steps[0], dsteps[0]
    rows = np.nonzero(st.q_lens == 1)[0]
    tok = st.query_start_loc[rows]
    q = d["q"][torch.from_numpy(tok.astype(np.int64)).to(dev)].contiguous()
    # a batch of its own carries a table as wide as its longest row (the mixed step's table is as wide
    # as its long prompt, which would size the decode splits for that prompt)
    width = int((st.seq_lens[rows].max() + 15) // 16)
    bt = d["bt"][torch.from_numpy(rows.astype(np.int64)).to(dev)][:, :width].contiguous()
    sl = d["sl"][torch.from_numpy(rows.astype(np.int64)).to(dev)].contiguous()
    qsl = torch.arange(len(rows) + 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.zeros(max(pa.workspace_size(len(rows), len(rows), bt.shape[1], w.num_q_heads, kc, ks, vs), 256),
                     dtype=torch.uint8, device=dev)

    def call():
        pa.attention(q, kc, vc, bt, sl, qsl, w.scale, out, workspace=ws, window=win, k_scale=ks, v_scale=vs,
                     max_q_len=1)

    for _ in range(5):
        call()
    pa.timing_reset()
    pa.timing_enable(True)
    for _ in range(steps_n):
        call()
    torch.cuda.synchronize()
    ms, n = pa.timing_read("decode_split")
    mms, mn = pa.timing_read("decode_merge")
    pa.timing_enable(False)
    pa.timing_reset()
    return {"avg_us": 1e3 * ms / n, "merge_us": 1e3 * mms / mn if mn else 0.0}


# Compute-bound launches get faster over a run's first few dozen launches (the clock settles), so
# prefill workloads warm up for at least this many steps whatever --warmup says.
PREFILL_MIN_WARMUP = 60


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--window", type=int, default=0, help="sliding window in keys (0: none)")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "i8"], help="cache element type")
    ap.add_argument("--verify", type=int, default=0, help="tokens per request to verify (decode workloads)")
    ap.add_argument("--chunks", type=int, default=1,
                    help="c3: append and attend the prompt as this many equal chunks (a step = all of them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="time the named workload only (the default run adds c3, c4 and c5 entries)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="instead of the hot path, time a plain device copy of this many MiB "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the hot path here is single-GPU (no collectives); "
              "use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.window < 0:
        print("--window must be >= 0", file=sys.stderr)
        sys.exit(2)
    if args.kv == "i8" and args.config == "c1":
        print("--kv i8 serves the bf16-activation workloads (c2 .. c5)", file=sys.stderr)
        sys.exit(2)
    if args.verify > 1 and args.config not in ("c2", "c5"):
        print("--verify serves the decode workloads (c2, c5)", file=sys.stderr)
        sys.exit(2)
    if args.chunks < 1 or (args.chunks > 1 and args.config != "c3"):
        print("--chunks serves the one-shot prefill workload (c3)", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_paged_kv_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load_library()
    dev = torch.device("cuda:0")

    if args.copy_ref_mib:
        n = args.copy_ref_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_ref_bytes_read": n, "copy_ref_bytes_written": n, "ms_per_copy": dt * 1e3,
                          "GBps_read_plus_write": 2 * n / dt / 1e9}), flush=True)
        return


    def warm(cfg):
        return max(args.warmup, PREFILL_MIN_WARMUP) if cfg in ("c3", "c4") else args.warmup

    head = measure(args.config, args.kv, args.window, args.verify, args.steps, warm(args.config), dev,
                   want_cpu=not args.no_cpu_baseline, chunks=args.chunks)
    if head["cpu_baseline"] is not None:
        ncpu, model = host_cpu()
        head["cpu_baseline"].update({"host_cpus": ncpu, "cpu_model": model})
    others = {}
    default_run = (args.config == "c2" and args.kv == "bf16" and args.window == 0 and args.verify <= 1
                   and args.chunks == 1 and not args.only)
    if default_run:
        for cfg in ("c3", "c4", "c5"):
            rec = measure(cfg, "bf16", 0, 0, args.steps, warm(cfg), dev)
            rec.pop("cpu_baseline")
            others[cfg] = rec
        # the same 8192-token prompt in four 2048-token chunks (each re-reading the cached keys of the
        # ones before it), against the one-shot prefill: total GPU time per prompt
        rec = measure("c3", "bf16", 0, 0, max(1, args.steps // 4), warm("c3") // 4 + 1, dev, chunks=4)
        rec.pop("cpu_baseline")
        rec["chunked_over_one_shot"] = round(rec["gpu_ms_per_step"] / others["c3"]["gpu_ms_per_step"], 4)
        others["c3_chunks4"] = rec
    from attention_paged_kv_amd.sched import bench_planner
    planner = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in bench_planner().items()}

    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "gpu_ms_per_step": head["gpu_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "kernels": head["kernels"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "host_planner": planner,
    }
    for k in ("decode_part", "step_roofline_frac"):
        if k in head:
            res[k] = head[k]
    if head["warmup"] != args.warmup:
        res["warmup_run"] = head["warmup"]
    if others:
        res["workloads"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
