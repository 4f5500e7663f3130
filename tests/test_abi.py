"""CPU checks of the C-ABI library: it loads, exports every symbol pa.h declares, and rejects bad
arguments on the host before touching any device."""
import ctypes
import glob
import os
import re

import pytest

import attention_paged_kv_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        from attention_paged_kv_amd import build
        build.build()
    return pa.load_library()


def test_header_declares_the_two_hot_path_calls():
    names = declared_functions()
    assert "pa_append_kv" in names and "pa_attention" in names and "pa_sched_schedule" in names
    assert len(names) >= 18


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(pa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_abi_version(lib):
    assert lib.pa_abi_version() == pa.ABI_VERSION


def _desc(nb=8, bs=16, hkv=2, d=128, dtype=1):
    return pa._CacheDesc(nb, bs, hkv, d, dtype)


def test_workspace_size_is_host_only_and_bounded(lib):
    d = _desc()
    assert lib.pa_attention_workspace_size(4, 4, 16, 8, ctypes.byref(d)) > 0
    ws = lib.pa_attention_workspace_size(4, 4, 64, 8, ctypes.byref(d))
    # 64 blocks = 1024 keys = several decode splits: rows x splits x heads x (d + 2) fp32 partials
    assert ws >= 4 * 2 * 8 * 130 * 4
    assert lib.pa_attention_workspace_size(0, 4, 16, 8, ctypes.byref(d)) == 0      # no requests
    assert lib.pa_attention_workspace_size(4, 3, 16, 8, ctypes.byref(d)) == 0      # q_len < 1 somewhere
    assert lib.pa_attention_workspace_size(4, 4, 16, 7, ctypes.byref(d)) == 0      # Hq % Hkv != 0
    bad = _desc(bs=32)
    assert lib.pa_attention_workspace_size(4, 4, 16, 8, ctypes.byref(bad)) == 0


@pytest.mark.parametrize("field,val,code", [("block_size", 32, 1), ("head_dim", 96, 2), ("dtype", 7, 2),
                                            ("num_blocks", 0, 1), ("num_kv_heads", 0, 1)])
def test_bad_descriptor_rejected_before_launch(lib, field, val, code):
    d = _desc()
    setattr(d, field, val)
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    rc = lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(0.1), p, None, 0, None)
    assert rc == code
    assert lib.pa_last_error()
    rc = lib.pa_append_kv(p, p, p, 4, p, p, ctypes.byref(d), None)
    assert rc == code


def test_bad_sizes_rejected_before_launch(lib):
    d = _desc()
    p = ctypes.c_void_p(16)
    assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 0, 16, p, p, ctypes.c_float(1), p, None, 0, None) == 1
    assert lib.pa_attention(p, 3, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), p, None, 0, None) == 1
    assert lib.pa_attention(p, 4, 6, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), p, None, 0, None) == 1
    assert lib.pa_attention(None, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), p, None, 0, None) == 1
    assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(float("inf")), p, None, 0,
                            None) == 1
    for bad_scale in (0.0, -0.125):
        assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(bad_scale),
                                ctypes.c_void_p(48), None, 0, None) == 1
        assert b"scale" in lib.pa_last_error()
    small = ctypes.c_void_p(256)
    o = ctypes.c_void_p(48)
    assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), p, small, 8, None) == 1  # out aliases q
    # 64 blocks per request -> split partials need workspace; an 8-byte one is refused before any launch
    assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(d), p, 4, 64, p, p, ctypes.c_float(1), o, small, 8, None) == 4
    assert b"workspace" in lib.pa_last_error()
    assert lib.pa_append_kv(p, p, p, -1, p, p, ctypes.byref(d), None) == 1
    assert lib.pa_append_kv(None, None, None, 0, None, None, ctypes.byref(d), None) == 0     # empty append


def test_misaligned_buffers_rejected_before_launch(lib):
    d = _desc()
    p, o, c2, bad = (ctypes.c_void_p(x) for x in (16, 48, 4096, 4104))
    for args in ((bad, 4, 8, p, c2), (p, 4, 8, bad, c2), (p, 4, 8, p, bad)):
        q, T, H, kc, vc = args
        assert lib.pa_attention(q, T, H, kc, vc, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), o, None, 0,
                                None) == 1
        assert b"aligned" in lib.pa_last_error()
    assert lib.pa_attention(p, 4, 8, p, c2, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), bad, None, 0,
                            None) == 1
    assert lib.pa_attention(p, 4, 8, p, c2, ctypes.byref(d), p, 4, 64, p, p, ctypes.c_float(1), o, bad, 1 << 20,
                            None) == 1
    assert lib.pa_append_kv(bad, p, p, 4, o, c2, ctypes.byref(d), None) == 1
    assert lib.pa_append_kv(p, p, p, 4, o, bad, ctypes.byref(d), None) == 1
    i8 = pa._CacheDesc(8, 16, 2, 128, 2, c2, bad)
    assert lib.pa_append_kv(p, p, p, 4, o, c2, ctypes.byref(i8), None) == 1
    assert b"aligned" in lib.pa_last_error()


def test_window_option_rejected_when_negative_before_launch(lib):
    d = _desc()
    p = ctypes.c_void_p(16)
    o = ctypes.c_void_p(48)
    neg = pa._AttnOpts(-1)
    rc = lib.pa_attention_ex(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), o, None, 0,
                             ctypes.byref(neg), None)
    assert rc == 1 and b"sliding_window" in lib.pa_last_error()
    negq = pa._AttnOpts(0, -1)
    rc = lib.pa_attention_ex(p, 4, 8, p, p, ctypes.byref(d), p, 4, 16, p, p, ctypes.c_float(1), o, None, 0,
                             ctypes.byref(negq), None)
    assert rc == 1 and b"max_q_len" in lib.pa_last_error()
    # a window does not lift the other checks: the 8-byte workspace is still refused before launch
    win = pa._AttnOpts(1000)     # rows may span 1015 keys: 4 splits, partials in the workspace
    small = ctypes.c_void_p(256)
    assert lib.pa_attention_ex(p, 4, 8, p, p, ctypes.byref(d), p, 4, 64, p, p, ctypes.c_float(1), o, small, 8,
                               ctypes.byref(win), None) == 4


def test_int8_descriptor_rules_checked_before_launch(lib):
    p = ctypes.c_void_p(16)
    o = ctypes.c_void_p(48)
    sc = ctypes.c_void_p(4096)
    no_scales = _desc(dtype=2)
    rc = lib.pa_attention(p, 4, 8, p, p, ctypes.byref(no_scales), p, 4, 16, p, p, ctypes.c_float(1), o, None, 0, None)
    assert rc == 1 and b"k_scale" in lib.pa_last_error()
    assert lib.pa_append_kv(p, p, p, 4, p, p, ctypes.byref(no_scales), None) == 1
    stray = pa._CacheDesc(8, 16, 2, 128, 1, sc, sc)          # scales on a bf16 cache
    assert lib.pa_attention(p, 4, 8, p, p, ctypes.byref(stray), p, 4, 16, p, p, ctypes.c_float(1), o, None, 0,
                            None) == 1
    i8 = pa._CacheDesc(8, 16, 2, 128, 2, sc, sc)
    # rows of up to 64 blocks take several decode splits, whose partials need workspace: an 8-byte
    # one is refused before launch
    assert lib.pa_attention(p, 13, 8, p, p, ctypes.byref(i8), p, 4, 64, p, p, ctypes.c_float(1), o,
                            ctypes.c_void_p(256), 8, None) == 4
    assert lib.pa_attention_workspace_size(4, 4, 64, 8, ctypes.byref(i8)) > 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        saved = pa._lib
        pa._lib = None
        try:
            pa.load_library(str(tmp_path / "missing.so"))
        finally:
            pa._lib = saved


@pytest.mark.parametrize("dtype", [1, 2])
@pytest.mark.parametrize("window,max_q", [(0, 0), (8000, 0), (4096, 0), (100, 0), (8000, 8), (0, 2)])
def test_workspace_size_serves_every_option(lib, window, max_q, dtype):
    """pa_attention_workspace_size() for the sizes bounds what any window and q_len bound needs: a
    call given exactly that many bytes is never refused for its workspace (code 4).  Rows of up to
    8208 keys sit where the split length changes with the window (256 or, over an 8-bit cache, 320
    keys vs 384)."""
    d = _desc(dtype=dtype)
    if dtype == 2:                      # an 8-bit cache needs scale pointers (never read on the host)
        d.k_scale = ctypes.c_void_p(512)
        d.v_scale = ctypes.c_void_p(768)
    p = ctypes.c_void_p(16)
    o = ctypes.c_void_p(48)
    for B, T in ((4, 4), (4, 20), (32, 32)):
        need = lib.pa_attention_workspace_size(B, T, 513, 8, ctypes.byref(d))
        assert need > 0
        opts = pa._AttnOpts(window, max_q)
        rc = lib.pa_attention_ex(p, T, 8, p, p, ctypes.byref(d), p, B, 513, p, p, ctypes.c_float(1), o,
                                 ctypes.c_void_p(256), need, ctypes.byref(opts), None)
        assert rc != 4, (B, T, window, max_q, lib.pa_last_error())


def test_noalloc_refuses_batches_beyond_its_scratch_on_the_host(lib):
    """pa_attention_noalloc sizes the call from the arguments alone and refuses a batch whose
    workspace exceeds its fixed scratch before touching any device (the pointers are never read)."""
    p = ctypes.c_void_p(16)
    o = ctypes.c_void_p(48)
    d = _desc(nb=4096, hkv=8, dtype=1)
    # 31 requests over 2078 query tokens and 1920-block rows: split partials for up to 8 positions
    # per row over 30720 keys, far more than 64 MiB
    need = lib.pa_attention_workspace_size(31, 2078, 1920, 32, ctypes.byref(d))
    assert need > (64 << 20)
    rc = lib.pa_attention_noalloc(p, 2078, 32, p, p, ctypes.byref(d), p, 31, 1920, p, p, ctypes.c_float(0.1), o,
                                  None, None)
    assert rc == 4 and b"scratch" in lib.pa_last_error()
