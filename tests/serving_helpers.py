"""Driver of a multi-step serving run for the tests: the host step planner (libpa pa_sched_*) plans
each step, an executor appends and attends, and each step is checked against the oracle run from
scratch on a fresh contiguous cache per request.

Synthetic K, V and Q of a token are a deterministic function of its whole token prefix (a 64-bit
chain hash seeds the draw), as a model's would be, so reusing a cached block is valid exactly when
the prefix matches.  Sampled tokens are a function of the last prefix hash.
"""
import numpy as np

from attention_paged_kv_amd import workloads as W
from attention_paged_kv_amd.sched import Planner
import oracle

HQ, HKV, D = 8, 2, 128
MASK = (1 << 64) - 1


def chain(h, tok):
    return (h * 6364136223846793005 + tok * 1442695040888963407 + 1) & MASK


class Tokens:
    """Per-request token ids, prefix hashes and the synthetic q/k/v rows they imply."""

    def __init__(self):
        self.toks = {}
        self.hashes = {}
        self.rows = {}

    def add(self, rid, prompt):
        self.toks[rid] = list(prompt)
        self.hashes[rid] = []

    def hash_at(self, rid, p):
        hs = self.hashes[rid]
        while len(hs) <= p:
            hs.append(chain(hs[-1] if hs else 0x1234567, self.toks[rid][len(hs)]))
        return hs[p]

    def qkv(self, rid, p):
        h = self.hash_at(rid, p)
        if h not in self.rows:
            x = np.random.default_rng(h).standard_normal((HQ + 2 * HKV) * D, dtype=np.float32)
            b = W.f32_to_bf16_bits(x)
            self.rows[h] = (b[:HQ * D].reshape(HQ, D), b[HQ * D:(HQ + HKV) * D].reshape(HKV, D),
                            b[(HQ + HKV) * D:].reshape(HKV, D))
        return self.rows[h]


def reference_step(tk, b, scale):
    """Oracle over a fresh cache: each request's context rows regenerated from its prefix hashes."""
    B = b.num_seqs
    seq = b.seq_lens.astype(np.int64)
    ql = np.diff(b.query_start_loc).astype(np.int64)
    nblk = (seq + 15) // 16
    NB = int(nblk.sum()) + 1
    MB = int(nblk.max())
    kc = np.zeros((NB, 16, HKV, D), np.uint16)
    vc = np.zeros((NB, 16, HKV, D), np.uint16)
    tables = np.full((B, MB), -1, np.int32)
    off = 0
    for i in range(B):
        tables[i, :nblk[i]] = np.arange(off, off + nblk[i])
        off += nblk[i]
    q = np.zeros((b.num_tokens, HQ, D), np.uint16)
    kn = np.zeros((b.num_tokens, HKV, D), np.uint16)
    vn = np.zeros_like(kn)
    slots = np.zeros(b.num_tokens, np.int32)
    for i in range(B):
        rid = int(b.request_ids[i])
        ctx = int(seq[i] - ql[i])
        for p in range(ctx):
            _, k, v = tk.qkv(rid, p)
            kc[tables[i, p // 16], p % 16] = k
            vc[tables[i, p // 16], p % 16] = v
        for j in range(int(ql[i])):
            t = int(b.query_start_loc[i]) + j
            p = ctx + j
            q[t], kn[t], vn[t] = tk.qkv(rid, p)
            slots[t] = tables[i, p // 16] * 16 + p % 16
    oracle.append(kn, vn, slots, kc, vc)
    out, _ = oracle.attention(q, kc, vc, tables, seq.astype(np.int32), b.query_start_loc, scale)
    return q, kn, vn, out



def drive(seed, nb, budget, prefix, execute, check, steps=60, mb=16, max_seqs=8):
    """Runs the planner for `steps` steps; execute(batch, q, k, v) -> out (uint16 bf16 bits) runs the
    step on the executor's own paged cache; check(out, ref, step) compares.  Returns counters."""
    rng = np.random.default_rng(seed)
    planner = Planner(nb, mb, budget, max_seqs=max_seqs, prefix_cache=prefix)
    scale = 1.0 / np.sqrt(D)
    tk = Tokens()
    shared = [int(x) for x in rng.integers(0, 50, 70)]
    rid = 0
    preempts = done = 0
    for step in range(steps):
        if rng.random() < 0.45 and rid < 24:
            pre = shared[: int(rng.integers(0, 70))]
            prompt = pre + [int(x) for x in rng.integers(0, 50, int(rng.integers(1, 60)))]
            max_new = int(rng.integers(1, 25))
            if len(prompt) + max_new <= mb * 16:
                planner.add(rid, prompt, max_new)
                tk.add(rid, prompt)
                rid += 1
        b = planner.schedule()
        preempts += len(planner.preempted())
        if b.num_seqs == 0:
            planner.commit([])
            continue
        q, kn, vn, ref = reference_step(tk, b, scale)
        out = execute(b, q, kn, vn, scale)
        check(out, ref, step, b)
        nxt = []
        for i in range(b.num_seqs):
            r = int(b.request_ids[i])
            last = int(b.query_start_loc[i + 1]) - 1
            t = int(tk.hash_at(r, int(b.positions[last])) % 50)
            nxt.append(t)
            if b.samples[i]:
                tk.toks[r].append(t)
        planner.commit(nxt)
        done += 1
    return dict(steps=done, hits=planner.stats()["hit_tokens"], preempts=preempts)


class OraclePagedExecutor:
    """The oracle over the planner's own paged cache (the layout the GPU uses)."""

    def __init__(self, nb):
        self.kc = np.zeros((nb, 16, HKV, D), np.uint16)
        self.vc = np.zeros((nb, 16, HKV, D), np.uint16)

    def __call__(self, b, q, kn, vn, scale):
        oracle.append(kn, vn, b.slot_mapping, self.kc, self.vc)
        out, _ = oracle.attention(q, self.kc, self.vc, b.block_tables, b.seq_lens, b.query_start_loc, scale)
        return out
