"""CPU oracle for causal attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.  It is a ctypes wrapper over ``pa_oracle.c``
(plain C, fp64 accumulation, explicit block-table gather, explicit causal mask), which
shares no code with the HIP kernels.  Its parity is pinned by the CPU tests (library dense
causal softmax on tiny inputs, closed forms, argmax probes, page invariants).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
F32, BF16, I8 = 0, 1, 2


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P, I, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
        lib.pa_oracle_append.argtypes = [P, P, P, I, P, P, I, I, I, I, ctypes.c_char_p, I]
        lib.pa_oracle_append.restype = I
        lib.pa_oracle_append_i8.argtypes = [P, P, P, I, P, P, I, I, I, P, P, ctypes.c_char_p, I]
        lib.pa_oracle_append_i8.restype = I
        lib.pa_oracle_quantize.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.pa_oracle_quantize.restype = ctypes.c_int
        lib.pa_oracle_attention.argtypes = [P, I, I, P, P, I, I, I, I, I, P, P, P, I, I, P, P, D, I, P, I, P, P, I,
                                            ctypes.c_char_p, I]
        lib.pa_oracle_attention.restype = I
        lib.pa_oracle_f64_to_bf16.argtypes = [D]
        lib.pa_oracle_f64_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def f64_to_bf16(x: float) -> int:
    return int(_load().pa_oracle_f64_to_bf16(float(x)))


def quantize(x: float, s: float) -> int:
    """int8 code of one float32 value under scale s."""
    return int(_load().pa_oracle_quantize(float(x), float(s)))


def _scales(a, Hkv, d):
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert a.shape == (Hkv, d)
    return a


def append(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None):
    """Write each token's K/V row into the cache slot given for it (in place on the caches): a copy,
    or for int8 caches the per-(head, channel) quantisation of the bf16 rows."""
    lib = _load()
    for a in (k, v, k_cache, v_cache):
        assert a.flags.c_contiguous
    NB, bs, Hkv, d = k_cache.shape
    assert bs == 16
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    err = ctypes.create_string_buffer(256)
    if k_cache.dtype == np.int8:
        assert v_cache.dtype == np.int8 and k.dtype == np.uint16 and v.dtype == np.uint16
        ks, vs = _scales(k_scale, Hkv, d), _scales(v_scale, Hkv, d)
        rc = lib.pa_oracle_append_i8(_ptr(k), _ptr(v), _ptr(slot_mapping), int(slot_mapping.shape[0]),
                                     _ptr(k_cache), _ptr(v_cache), NB, Hkv, d, _ptr(ks), _ptr(vs), err, 256)
        if rc != 0:
            raise OracleError(err.value.decode())
        return
    assert k_cache.dtype == k.dtype and v_cache.dtype == v.dtype
    rc = lib.pa_oracle_append(_ptr(k), _ptr(v), _ptr(slot_mapping), int(slot_mapping.shape[0]), _ptr(k_cache),
                              _ptr(v_cache), NB, Hkv, d, k.dtype.itemsize, err, 256)
    if rc != 0:
        raise OracleError(err.value.decode())


def attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale, rows=None,
              want_f64=False, num_threads=None, window=0, k_scale=None, v_scale=None):
    """Causal attention of every (or the listed) query token row over its request's paged keys
    (with ``window`` > 0, only each row's ``window`` most recent keys).

    Returns (out, out_f64): ``out`` in the storage dtype of ``q`` (float32 or uint16 bf16 bits),
    ``out_f64`` the unrounded double result (or None).  Rows not computed are left zero.  int8
    caches (with bf16 ``q``) are read as code * scale of their (head, channel).
    """
    lib = _load()
    dtype = F32 if q.dtype == np.float32 else BF16
    assert q.dtype in (np.float32, np.uint16)
    q = np.ascontiguousarray(q)
    T, Hq, d = q.shape
    NB, bs, Hkv, d2 = k_cache.shape
    assert bs == 16 and d2 == d
    cache_dtype = I8 if k_cache.dtype == np.int8 else dtype
    ks = vs = None
    if cache_dtype == I8:
        ks, vs = _scales(k_scale, Hkv, d), _scales(v_scale, Hkv, d)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    query_start_loc = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    B, MB = block_tables.shape
    out = np.zeros_like(q)
    out64 = np.zeros(q.shape, dtype=np.float64) if want_f64 else None
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    nt = int(num_threads or default_threads())
    err = ctypes.create_string_buffer(256)
    rc = lib.pa_oracle_attention(_ptr(q), T, Hq, _ptr(np.ascontiguousarray(k_cache)),
                                 _ptr(np.ascontiguousarray(v_cache)), NB, Hkv, d, dtype, cache_dtype, _ptr(ks),
                                 _ptr(vs), _ptr(block_tables), B, MB,
                                 _ptr(seq_lens), _ptr(query_start_loc), float(scale), int(window), _ptr(rows_a),
                                 0 if rows_a is None else int(rows_a.shape[0]), _ptr(out), _ptr(out64), nt, err, 256)
    if rc != 0:
        raise OracleError(err.value.decode())
    return out, out64


def run_step(w, step, k_cache, v_cache, rows=None, want_f64=False, num_threads=None, window=0):
    """Append the step's K/V into (k_cache, v_cache) in place, then attend; returns (out, out_f64)."""
    ks, vs = getattr(w, "k_scale", None), getattr(w, "v_scale", None)
    append(step.k_new, step.v_new, step.slot_mapping, k_cache, v_cache, ks, vs)
    return attention(step.q, k_cache, v_cache, step.block_tables, step.seq_lens, step.query_start_loc, w.scale,
                     rows=rows, want_f64=want_f64, num_threads=num_threads, window=window, k_scale=ks, v_scale=vs)
