"""Host step planner of libpa (include/pa_sched.h): block pool, token-budget scheduler, prefix cache.

A thin ctypes binding: every decision is made by the C++ planner; this module only owns the host
arrays a step is written into.

    p = Planner(num_blocks, max_blocks_per_seq, token_budget, max_seqs=0, prefix_cache=True)
    p.add(request_id, prompt_token_ids, max_new_tokens)
    b = p.schedule()          # Batch: request_ids, query_start_loc, seq_lens, block_tables,
                              #        slot_mapping, token_ids, positions, samples (numpy views)
    ... append this step's K/V at b.slot_mapping, run attention with b's index arrays ...
    p.commit(next_tokens, stop=None)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import PAError, load_library

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class _Config(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("token_budget", ctypes.c_int32), ("max_seqs", ctypes.c_int32), ("prefix_cache", ctypes.c_int32)]


class _Batch(ctypes.Structure):
    _fields_ = [("cap_seqs", ctypes.c_int32), ("cap_tokens", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("num_tokens", ctypes.c_int32), ("request_ids", _I64P), ("query_start_loc", _I32P),
                ("seq_lens", _I32P), ("block_tables", _I32P), ("slot_mapping", _I32P), ("token_ids", _I32P),
                ("positions", _I32P), ("samples", _I32P)]


class _Stats(ctypes.Structure):
    _fields_ = [("free_blocks", ctypes.c_int32), ("cached_blocks", ctypes.c_int32),
                ("evictable_blocks", ctypes.c_int32), ("running", ctypes.c_int32), ("waiting", ctypes.c_int32),
                ("preempted_last_step", ctypes.c_int32), ("hit_tokens", ctypes.c_int64)]


_ready = False


def _lib():
    global _ready
    lib = load_library()
    if not _ready:
        P = ctypes.c_void_p
        I = ctypes.c_int32
        lib.pa_sched_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(P)]
        lib.pa_sched_create.restype = ctypes.c_int
        lib.pa_sched_destroy.argtypes = [P]
        lib.pa_sched_destroy.restype = None
        lib.pa_sched_add.argtypes = [P, ctypes.c_int64, _I32P, I, I]
        lib.pa_sched_add.restype = ctypes.c_int
        lib.pa_sched_abort.argtypes = [P, ctypes.c_int64]
        lib.pa_sched_abort.restype = ctypes.c_int
        lib.pa_sched_schedule.argtypes = [P, ctypes.POINTER(_Batch)]
        lib.pa_sched_schedule.restype = ctypes.c_int
        lib.pa_sched_commit.argtypes = [P, _I32P, _I32P]
        lib.pa_sched_commit.restype = ctypes.c_int
        lib.pa_sched_get_stats.argtypes = [P, ctypes.POINTER(_Stats)]
        lib.pa_sched_get_stats.restype = ctypes.c_int
        lib.pa_sched_preempted.argtypes = [P, _I64P, I, ctypes.POINTER(I)]
        lib.pa_sched_preempted.restype = ctypes.c_int
        _ready = True
    return lib


def _check(lib, rc):
    if rc != 0:
        raise PAError(rc, lib.pa_last_error().decode(errors="replace"))


@dataclass
class Batch:
    request_ids: np.ndarray      # [B] int64
    query_start_loc: np.ndarray  # [B+1] int32
    seq_lens: np.ndarray         # [B] int32
    block_tables: np.ndarray     # [B, max_blocks_per_seq] int32, -1 padded
    slot_mapping: np.ndarray     # [T] int32
    token_ids: np.ndarray        # [T] int32
    positions: np.ndarray        # [T] int32
    samples: np.ndarray          # [B] int32

    @property
    def num_seqs(self) -> int:
        return int(self.request_ids.shape[0])

    @property
    def max_q_len(self) -> int:
        """Longest q_len of the step: the bound to pass as attention(..., max_q_len=)."""
        return int(np.diff(self.query_start_loc).max()) if self.num_seqs else 0

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])


class Planner:
    def __init__(self, num_blocks, max_blocks_per_seq, token_budget, max_seqs=0, prefix_cache=True):
        self._l = _lib()
        cfg = _Config(num_blocks, max_blocks_per_seq, token_budget, max_seqs, 1 if prefix_cache else 0)
        h = ctypes.c_void_p()
        _check(self._l, self._l.pa_sched_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        self.mb = max_blocks_per_seq
        self.token_budget = token_budget
        self.max_seqs = max_seqs
        self._live = 0
        self._last = 0

    def close(self):
        if self._h:
            self._l.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, request_id, prompt, max_new_tokens):
        a = np.ascontiguousarray(prompt, dtype=np.int32)
        _check(self._l, self._l.pa_sched_add(self._h, int(request_id), a.ctypes.data_as(_I32P), int(a.shape[0]),
                                             int(max_new_tokens)))
        self._live += 1

    def abort(self, request_id):
        _check(self._l, self._l.pa_sched_abort(self._h, int(request_id)))

    def _buffers(self, cap_s):
        """Host arrays the planner writes into, kept across steps and grown when needed."""
        if getattr(self, "_cap_s", 0) < cap_s:
            cap_s = max(cap_s, 2 * getattr(self, "_cap_s", 0))
            cap_t = self.token_budget
            self._arr = dict(ids=np.zeros(cap_s, np.int64), qsl=np.zeros(cap_s + 1, np.int32),
                             sl=np.zeros(cap_s, np.int32), bt=np.zeros((cap_s, self.mb), np.int32),
                             slots=np.zeros(cap_t, np.int32), toks=np.zeros(cap_t, np.int32),
                             pos=np.zeros(cap_t, np.int32), smp=np.zeros(cap_s, np.int32))
            a = self._arr
            self._batch = _Batch(cap_s, cap_t, 0, 0, a["ids"].ctypes.data_as(_I64P), a["qsl"].ctypes.data_as(_I32P),
                                 a["sl"].ctypes.data_as(_I32P), a["bt"].ctypes.data_as(_I32P),
                                 a["slots"].ctypes.data_as(_I32P), a["toks"].ctypes.data_as(_I32P),
                                 a["pos"].ctypes.data_as(_I32P), a["smp"].ctypes.data_as(_I32P))
            self._cap_s = cap_s
        return self._arr, self._batch

    def schedule(self) -> Batch:
        """Plans one step; the returned arrays are copies the caller may keep."""
        st = self.stats()
        a, b = self._buffers(self.max_seqs if self.max_seqs > 0 else max(1, st["running"] + st["waiting"]))
        _check(self._l, self._l.pa_sched_schedule(self._h, ctypes.byref(b)))
        n, t = b.num_seqs, b.num_tokens
        self._last = n
        return Batch(a["ids"][:n].copy(), a["qsl"][:n + 1].copy(), a["sl"][:n].copy(), a["bt"][:n].copy(),
                     a["slots"][:t].copy(), a["toks"][:t].copy(), a["pos"][:t].copy(), a["smp"][:n].copy())

    def schedule_views(self, cap_seqs):
        """Plans one step into the planner's own buffers (no copies; valid until the next call).
        Returns (num_seqs, num_tokens, arrays)."""
        a, b = self._buffers(cap_seqs)
        _check(self._l, self._l.pa_sched_schedule(self._h, ctypes.byref(b)))
        return b.num_seqs, b.num_tokens, a

    def commit(self, next_tokens, stop=None):
        nt = np.ascontiguousarray(next_tokens if len(next_tokens) else [0], dtype=np.int32)
        sp = None if stop is None else np.ascontiguousarray(stop, dtype=np.int32)
        _check(self._l, self._l.pa_sched_commit(self._h, nt.ctypes.data_as(_I32P),
                                                None if sp is None else sp.ctypes.data_as(_I32P)))

    def stats(self) -> dict:
        s = _Stats()
        _check(self._l, self._l.pa_sched_get_stats(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in _Stats._fields_}

    def preempted(self):
        n = ctypes.c_int32()
        buf = np.zeros(4096, np.int64)
        _check(self._l, self._l.pa_sched_preempted(self._h, buf.ctypes.data_as(_I64P), 4096, ctypes.byref(n)))
        return [int(x) for x in buf[:min(n.value, 4096)]]


def bench_planner(decodes=30, prompt=30000, budget=2048, wide=256, wide_ctx=2048):
    """Host cost of the C++ planner, in microseconds per schedule + commit (median over steps, the
    planner writing into preallocated host arrays), for two step shapes: P4's mixed step
    (`decodes` users decoding while a `prompt`-token prompt goes through in `budget`-token chunks)
    and a wide decode batch (`wide` requests of `wide_ctx` tokens)."""
    import time

    def timed_steps(p, cap, stop_when=None, n=None):
        nt = np.full(max(cap, 1), 7, np.int32)
        nt_p = nt.ctypes.data_as(_I32P)
        times, k = [], 0
        while True:
            t0 = time.perf_counter()
            ns, _, a = p.schedule_views(cap)
            _check(p._l, p._l.pa_sched_commit(p._h, nt_p, None))
            times.append(time.perf_counter() - t0)
            k += 1
            if (stop_when and stop_when(ns, a)) or (n and k == n):
                return 1e6 * float(np.median(times)), k

    out = {}
    p = Planner(8192, 4096, budget)
    for i in range(decodes):
        p.add(i, [1000 + i] * 8, 60000)
    timed_steps(p, 64, n=3)
    p.add(10 ** 6, list(range(prompt)), 4)
    big = lambda ns, a: any(a["ids"][j] == 10 ** 6 and a["smp"][j] == 1 for j in range(ns))
    out["mixed_chunked_us_per_step"], out["mixed_chunked_steps"] = timed_steps(p, 64, stop_when=big)
    mb = wide_ctx // 16 + 16
    q = Planner(wide * mb, mb, wide * 8)
    for i in range(wide):
        q.add(i, [i % 97 + 1] * wide_ctx, 200)
    while q.stats()["waiting"]:
        timed_steps(q, wide, n=1)
    timed_steps(q, wide, n=3)
    out["decode_batch_us_per_step"], _ = timed_steps(q, wide, n=50)
    out["decode_batch_seqs"] = wide
    return out
