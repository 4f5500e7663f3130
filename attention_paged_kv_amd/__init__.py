"""Paged-KV causal attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (the C ABI in ``include/pa.h``).  PyTorch supplies
device memory and the current stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or built for another ABI, calls raise.

    append_kv(k, v, slot_mapping, k_cache, v_cache)
    attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale, out, window=0)

Caches are ``[num_blocks, 16, num_kv_heads, head_dim]`` tensors (float32, bfloat16, or int8
codes with ``k_scale``/``v_scale`` float32 ``[num_kv_heads, head_dim]`` scales and bfloat16
activations), ``q``/``out`` are ``[num_tokens, num_q_heads, head_dim]``, indices are int32.
"""
from __future__ import annotations

import ctypes
import os

ABI_VERSION = 5
BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

_lib = None
_workspaces = {}


class PAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"pa error {code}: {msg}")
        self.code = code


class _CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


class _AttnOpts(ctypes.Structure):
    _fields_ = [("sliding_window", ctypes.c_int32), ("max_q_len", ctypes.c_int32)]


def load_library(path: str = LIB_PATH):
    """Load libpa.so and check its ABI version; raises if it is missing or mismatched."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m attention_paged_kv_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(_CacheDesc)
    lib.pa_abi_version.restype = ctypes.c_int
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_release.restype = None
    lib.pa_set_check.argtypes = [ctypes.c_int]
    lib.pa_set_check.restype = None
    lib.pa_append_kv.argtypes = [P, P, P, I, P, P, D, P]
    lib.pa_append_kv.restype = ctypes.c_int
    lib.pa_attention_workspace_size.argtypes = [I, I, I, I, D]
    lib.pa_attention_workspace_size.restype = Z
    lib.pa_attention.argtypes = [P, I, I, P, P, D, P, I, I, P, P, ctypes.c_float, P, P, Z, P]
    lib.pa_attention.restype = ctypes.c_int
    lib.pa_attention_ex.argtypes = [P, I, I, P, P, D, P, I, I, P, P, ctypes.c_float, P, P, Z,
                                    ctypes.POINTER(_AttnOpts), P]
    lib.pa_attention_ex.restype = ctypes.c_int
    lib.pa_attention_noalloc.argtypes = [P, I, I, P, P, D, P, I, I, P, P, ctypes.c_float, P,
                                         ctypes.POINTER(_AttnOpts), P]
    lib.pa_attention_noalloc.restype = ctypes.c_int
    lib.pa_timing_enable.argtypes = [ctypes.c_int]
    lib.pa_timing_enable.restype = ctypes.c_int
    lib.pa_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.pa_timing_read.restype = ctypes.c_int
    lib.pa_timing_reset.restype = None
    v = lib.pa_abi_version()
    if v != ABI_VERSION:
        raise ImportError(f"libpa ABI version {v} != binding version {ABI_VERSION}")
    _lib = lib
    return lib


def _err(lib, rc):
    if rc != 0:
        raise PAError(rc, lib.pa_last_error().decode(errors="replace"))


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.int8:
        return 2
    raise TypeError(f"unsupported cache dtype {t.dtype} (float32, bfloat16 or int8)")


def _act_dtype(k_cache):
    """dtype of q, k, v and out for this cache."""
    import torch
    return torch.bfloat16 if k_cache.dtype == torch.int8 else k_cache.dtype


def _check_tensor(name, t, device, dtype=None, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _desc(k_cache, k_scale=None, v_scale=None):
    import torch
    nb, bs, hkv, d = k_cache.shape
    if bs != BLOCK_SIZE:
        raise ValueError(f"cache block size must be {BLOCK_SIZE}, got {bs}")
    code = _dtype_code(k_cache)
    if code == 2:
        if k_scale is None or v_scale is None:
            raise ValueError("an int8 cache needs k_scale and v_scale")
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            _check_tensor(name, t, k_cache.device, dtype=torch.float32, ndim=2)
            if tuple(t.shape) != (hkv, d):
                raise ValueError(f"{name} must be [{hkv}, {d}], got {tuple(t.shape)}")
        return _CacheDesc(nb, bs, hkv, d, code, k_scale.data_ptr(), v_scale.data_ptr())
    if k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale are for int8 caches only")
    return _CacheDesc(nb, bs, hkv, d, code)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def append_kv(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None):
    """Write each token's K/V row ([T, Hkv, d]) to cache slot slot_mapping[t] (negative = skip);
    int8 caches store the per-(head, channel) quantised codes of the bf16 rows."""
    import torch
    lib = load_library()
    dev = k_cache.device
    _check_tensor("k_cache", k_cache, dev, ndim=4)
    _check_tensor("v_cache", v_cache, dev, dtype=k_cache.dtype, ndim=4)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _check_tensor("k", k, dev, dtype=_act_dtype(k_cache), ndim=3)
    _check_tensor("v", v, dev, dtype=_act_dtype(k_cache), ndim=3)
    _check_tensor("slot_mapping", slot_mapping, dev, dtype=torch.int32, ndim=1)
    T = k.shape[0]
    if v.shape != k.shape or tuple(k.shape[1:]) != tuple(k_cache.shape[2:]) or slot_mapping.shape[0] != T:
        raise ValueError("k/v must be [T, Hkv, d] matching the cache, slot_mapping [T]")
    desc = _desc(k_cache, k_scale, v_scale)
    rc = lib.pa_append_kv(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), T, k_cache.data_ptr(),
                          v_cache.data_ptr(), ctypes.byref(desc), _stream(dev))
    _err(lib, rc)


def workspace_size(num_seqs, num_q_tokens, max_blocks_per_seq, num_q_heads, k_cache, k_scale=None,
                   v_scale=None) -> int:
    lib = load_library()
    desc = _desc(k_cache, k_scale, v_scale)
    return int(lib.pa_attention_workspace_size(num_seqs, num_q_tokens, max_blocks_per_seq, num_q_heads,
                                               ctypes.byref(desc)))


def _workspace(dev, nbytes):
    """The binding's cached workspace for (device, current stream): calls queued on one stream run
    in order, so they may share one buffer; calls on different streams get different buffers."""
    import torch
    stream = torch.cuda.current_stream(dev)
    key = (dev.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        # allocated while `stream` is current, so the caching allocator ties the block to it
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale, out, workspace=None,
              window=0, k_scale=None, v_scale=None, max_q_len=0):
    """Causal attention of the varlen batch over the paged cache; writes ``out`` in place.

    ``window`` > 0 restricts each query row to its ``window`` most recent keys (pa_attention_ex);
    ``max_q_len`` > 0 promises that no request has a longer q_len (lets decode and verification
    steps skip the prefill-tile pass); int8 caches take their ``k_scale``/``v_scale``."""
    import torch
    lib = load_library()
    dev = q.device
    _check_tensor("q", q, dev, ndim=3)
    _check_tensor("k_cache", k_cache, dev, ndim=4)
    _check_tensor("v_cache", v_cache, dev, dtype=k_cache.dtype, ndim=4)
    if q.dtype != _act_dtype(k_cache):
        raise TypeError(f"q must be {_act_dtype(k_cache)} for a {k_cache.dtype} cache, got {q.dtype}")
    _check_tensor("out", out, dev, dtype=q.dtype, ndim=3)
    _check_tensor("block_tables", block_tables, dev, dtype=torch.int32, ndim=2)
    _check_tensor("seq_lens", seq_lens, dev, dtype=torch.int32, ndim=1)
    _check_tensor("query_start_loc", query_start_loc, dev, dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    T, Hq, d = q.shape
    B, MB = block_tables.shape
    if out.shape != q.shape or d != k_cache.shape[3]:
        raise ValueError("out must match q, head_dim must match the cache")
    if seq_lens.shape[0] != B or query_start_loc.shape[0] != B + 1:
        raise ValueError("seq_lens must be [B], query_start_loc [B+1]")
    desc = _desc(k_cache, k_scale, v_scale)
    opts = _AttnOpts(int(window), int(max_q_len))
    need = int(lib.pa_attention_workspace_size(B, T, MB, Hq, ctypes.byref(desc)))
    if need == 0:
        _err(lib, lib.pa_attention_ex(None, T, Hq, None, None, ctypes.byref(desc), None, B, MB, None, None,
                                      ctypes.c_float(scale), None, None, 0, ctypes.byref(opts), None))
    if workspace is None:
        workspace = _workspace(dev, need)
    _check_tensor("workspace", workspace, dev)
    rc = lib.pa_attention_ex(q.data_ptr(), T, Hq, k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(desc),
                             block_tables.data_ptr(), B, MB, seq_lens.data_ptr(), query_start_loc.data_ptr(),
                             ctypes.c_float(scale), out.data_ptr(), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), ctypes.byref(opts), _stream(dev))
    _err(lib, rc)
    return out


def attention_noalloc(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale, out, window=0,
                      k_scale=None, v_scale=None, max_q_len=0):
    """``attention`` through pa_attention_noalloc: the library's fixed per-device scratch array
    instead of a workspace, so the call allocates no device memory.  Calls that may overlap on
    one device race on that array (serialise them).  Raises PAError (code 4) for a batch whose
    workspace would not fit the array."""
    import torch
    lib = load_library()
    dev = q.device
    _check_tensor("q", q, dev, ndim=3)
    _check_tensor("k_cache", k_cache, dev, ndim=4)
    _check_tensor("v_cache", v_cache, dev, dtype=k_cache.dtype, ndim=4)
    if q.dtype != _act_dtype(k_cache):
        raise TypeError(f"q must be {_act_dtype(k_cache)} for a {k_cache.dtype} cache, got {q.dtype}")
    _check_tensor("out", out, dev, dtype=q.dtype, ndim=3)
    _check_tensor("block_tables", block_tables, dev, dtype=torch.int32, ndim=2)
    _check_tensor("seq_lens", seq_lens, dev, dtype=torch.int32, ndim=1)
    _check_tensor("query_start_loc", query_start_loc, dev, dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    T, Hq, d = q.shape
    B, MB = block_tables.shape
    if out.shape != q.shape or d != k_cache.shape[3]:
        raise ValueError("out must match q, head_dim must match the cache")
    if seq_lens.shape[0] != B or query_start_loc.shape[0] != B + 1:
        raise ValueError("seq_lens must be [B], query_start_loc [B+1]")
    desc = _desc(k_cache, k_scale, v_scale)
    opts = _AttnOpts(int(window), int(max_q_len))
    rc = lib.pa_attention_noalloc(q.data_ptr(), T, Hq, k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(desc),
                                  block_tables.data_ptr(), B, MB, seq_lens.data_ptr(), query_start_loc.data_ptr(),
                                  ctypes.c_float(scale), out.data_ptr(), ctypes.byref(opts), _stream(dev))
    _err(lib, rc)
    return out


def set_check(on: bool):
    """Validate index arguments on the device before each call (synchronises; for debugging)."""
    load_library().pa_set_check(1 if on else 0)


def timing_enable(on: bool):
    load_library().pa_timing_enable(1 if on else 0)


def timing_read(name: str):
    """(total milliseconds, launches) of a kernel family since the last reset."""
    lib = load_library()
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _err(lib, lib.pa_timing_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timing_reset():
    load_library().pa_timing_reset()


def release():
    load_library().pa_release()
    _workspaces.clear()
