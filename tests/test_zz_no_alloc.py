"""GPU test of pa_attention_noalloc, the entry point for callers that cannot allocate device memory:
through the C ABI it must give exactly what pa_attention_ex gives (same kernels, scratch in the
library's fixed per-device array instead of a workspace), and both must match the oracle.  Two
calls in a row, the second on a smaller batch, so the second reuses scratch the first left
behind."""
import numpy as np
import pytest
import torch

import attention_paged_kv_amd as pa
from attention_paged_kv_amd import workloads as W
import oracle
from tests.gpu_helpers import GpuState, compare, host_array, int_tensor, say

pytestmark = pytest.mark.gpu


def both_paths(w, window=0, max_q_len=0):
    """(no-alloc output, pa_attention_ex output, oracle output) of the workload's single step."""
    st = w.steps[0]
    g = GpuState(w)
    x = g.inputs(st)
    pa.append_kv(x["k"], x["v"], x["slots"], g.kc, g.vc, g.ks, g.vs)
    out_n = torch.full_like(x["q"], float("nan"))
    pa.attention_noalloc(x["q"], g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out_n, window=window,
                         k_scale=g.ks, v_scale=g.vs, max_q_len=max_q_len)
    torch.cuda.synchronize()
    ws = torch.empty(pa.workspace_size(st.num_seqs, st.num_tokens, st.block_tables.shape[1], w.num_q_heads,
                                       g.kc, g.ks, g.vs), dtype=torch.uint8, device=g.kc.device)
    out_e = torch.full_like(x["q"], float("nan"))
    pa.attention(x["q"], g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out_e, workspace=ws, window=window,
                 k_scale=g.ks, v_scale=g.vs, max_q_len=max_q_len)
    torch.cuda.synchronize()
    ref, _ = oracle.run_step(w, st, w.k_cache0.copy(), w.v_cache0.copy(), window=window)
    return host_array(out_n, w.dtype), host_array(out_e, w.dtype), ref


@pytest.mark.timeout(600)
def test_noalloc_equals_attention_ex_two_calls_second_smaller():
    # first: the long skewed decode batch (16 requests up to 32768 keys, 86 splits per row: about
    # 23 MB of split partials); second: a smaller mixed batch with decode rows, a verify row and a
    # prompt (stream-mode partials and the tile list), with a window
    big = W.config5()
    small = W.make_batch(91, [700, 90, 1300, 300, 40], [1, 1, 5, 200, 1], 16, 4, 128, "bf16", num_blocks=180)
    for name, w, window in (("c5 skewed decode", big, 0), ("small mixed batch, window 100", small, 100)):
        say(f"noalloc: {name}")
        got, ex, ref = both_paths(w, window=window)
        assert np.array_equal(got, ex), f"{name}: no-alloc output differs from pa_attention_ex"
        compare(got, ref, w.dtype, what=f"noalloc {name}")


def test_noalloc_int8_and_f32_batches():
    cases = [("int8 cache", W.make_batch(92, [900, 33, 120], [1, 1, 120], 8, 2, 128, "bf16", num_blocks=80,
                                         cache="i8")),
             ("f32", W.make_batch(93, [400, 77], [40, 1], 4, 2, 64, "f32", num_blocks=40))]
    for name, w in cases:
        got, ex, ref = both_paths(w)
        assert np.array_equal(got, ex), f"{name}: no-alloc output differs from pa_attention_ex"
        compare(got, ref, w.dtype, what=f"noalloc {name}")


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    """The mixed chunked step sizes ~0.5 GB of partials (rows of up to 8 positions over 30720
    keys): refused on the host with PA_ERR_WORKSPACE, nothing launched, output untouched."""
    w = W.config4(values=False)
    st = w.steps[0]
    dev = "cuda:0"
    T = int(st.query_start_loc[-1])             # values=False leaves q empty: take T from the offsets
    q = torch.zeros((T, 32, 128), dtype=torch.bfloat16, device=dev)
    # a cache of the workload's whole pool: every index of the call is valid even if it ran
    kc = torch.zeros((w.num_blocks, 16, 8, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PAError) as e:
        pa.attention_noalloc(q, kc, vc, int_tensor(st.block_tables), int_tensor(st.seq_lens),
                             int_tensor(st.query_start_loc), w.scale, out)
    assert e.value.code == 4 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_check_mode_reports_through_the_scratch_array():
    w = W.make_batch(94, [40], [1], 2, 2, 128, "bf16", num_blocks=4)
    st = w.steps[0]
    g = GpuState(w)
    x = g.inputs(st)
    bt = st.block_tables.copy()
    bt[0, 1] = 99
    out = torch.empty_like(x["q"])
    pa.set_check(True)
    try:
        with pytest.raises(pa.PAError) as e:
            pa.attention_noalloc(x["q"], g.kc, g.vc, int_tensor(bt), x["sl"], x["qsl"], w.scale, out)
        assert e.value.code == 5 and "block id" in str(e.value)
    finally:
        pa.set_check(False)
