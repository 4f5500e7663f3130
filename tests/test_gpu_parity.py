"""GPU parity: the library's HIP path (through its C ABI) against the CPU oracle.

Append must match bit for bit over the whole cache; attention within max-abs 2e-2 (bf16) or 1e-5
(fp32) plus a per-row relative-L2 gate; probes and invariance checks are bitwise.
"""
import numpy as np
import pytest
import torch

import attention_paged_kv_amd as pa
from attention_paged_kv_amd import workloads as W
import oracle
from tests.gpu_helpers import DEV, GpuState, compare, dev_tensor, host_array, int_tensor, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def check_mode():
    pa.set_check(True)
    yield
    pa.set_check(False)


def oracle_out(w, st, kc, vc, rows=None):
    out, _ = oracle.run_step(w, st, kc, vc, rows=rows)
    return out


def bits(a):
    """Raw bit patterns (NaN poison compares equal to itself)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a


def run_and_compare(w, rows=None, what=""):
    """One step on GPU and oracle; append compared bytewise, attention to tolerance."""
    st = w.steps[0]
    g = GpuState(w)
    out_g = g.step(st)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    out_r = oracle_out(w, st, kc, vc, rows=rows)
    assert np.array_equal(bits(host_array(g.kc, w.dtype)), bits(kc)), f"{what}: K cache differs after append"
    assert np.array_equal(bits(host_array(g.vc, w.dtype)), bits(vc)), f"{what}: V cache differs after append"
    compare(out_g, out_r, w.dtype, rows=rows, what=what)
    return out_g, out_r, g


# ------------------------------------------------------------------------------------------
# small ragged batches: decode rows, prefill tiles, chunks, GQA groups, both head dims / dtypes
# ------------------------------------------------------------------------------------------
SMALL = [
    # seq_lens, q_lens, Hq, Hkv, d, dtype
    ([1], [1], 1, 1, 64, "f32"),
    ([17], [17], 2, 2, 64, "f32"),
    ([300, 33, 16], [1, 1, 1], 4, 4, 128, "f32"),
    ([70, 129, 5], [70, 2, 5], 4, 2, 64, "f32"),
    ([1], [1], 1, 1, 128, "bf16"),
    ([2], [2], 8, 8, 128, "bf16"),
    ([15, 16, 17, 31, 32, 33], [1, 1, 1, 1, 1, 1], 8, 2, 128, "bf16"),
    ([255, 256, 257], [255, 256, 257], 4, 4, 128, "bf16"),
    ([1000, 513, 700], [1, 200, 64], 32, 8, 128, "bf16"),
    ([300, 47], [300, 1], 6, 3, 128, "bf16"),
    ([400, 129], [129, 129], 16, 1, 64, "bf16"),
    ([260, 90], [3, 90], 2, 2, 64, "bf16"),
    ([1030, 1030], [1, 7], 32, 32, 128, "bf16"),
    # bf16 head_dim 64 decode rows, one KV head: staged V rows are 128 bytes (8 chunks) wide
    ([15, 16, 17, 31, 32, 33, 700], [1, 1, 1, 1, 1, 1, 1], 8, 1, 64, "bf16"),
    ([300, 2000], [1, 1], 4, 4, 64, "bf16"),
    # more query heads per KV head than one MFMA holds: 32 (two column groups) and the maximum, 128
    ([3000, 77, 513], [1, 1, 1], 64, 2, 128, "bf16"),
    ([900, 20, 40], [1, 20, 3], 128, 1, 64, "bf16"),
    # a wide batch: 200 rows, lengths 1 .. 300, a few prompts among the decode rows
    ([1 + (37 * i) % 300 for i in range(200)], [1 if i % 50 else 1 + (37 * i) % 300 for i in range(200)],
     8, 8, 64, "bf16"),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_varlen_batches(case):
    seq, ql, Hq, Hkv, d, dt = SMALL[case]
    say(f"case {case}: seq {seq} q {ql} Hq {Hq} Hkv {Hkv} d {d} {dt}")
    nb = sum((s + 15) // 16 for s in seq) + 3
    w = W.make_batch(100 + case, seq, ql, Hq, Hkv, d, dt, num_blocks=nb)
    run_and_compare(w, what=f"small[{case}]")


@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1024, 2048])
def test_block_boundary_lengths(L):
    """Lengths on and around block multiples (P1 §4.3 reports a write bug that showed only when
    the length was a multiple of the block size)."""
    say(f"boundary L={L}")
    w = W.make_batch(200 + L, [L, L, L + 1], [L, 1, min(L, 17)], 8, 2, 128, "bf16")
    run_and_compare(w, what=f"boundary {L}")


# ------------------------------------------------------------------------------------------
# the five workloads
# ------------------------------------------------------------------------------------------
def test_c1_tiny_f32_prefill_then_decode():
    w = W.config1()
    g = GpuState(w)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    outs = []
    for i, st in enumerate(w.steps):
        og = g.step(st)
        orf = oracle_out(w, st, kc, vc)
        compare(og, orf, "f32", what=f"c1 step {i}")
        assert np.array_equal(bits(host_array(g.kc, "f32")), bits(kc))
        assert np.array_equal(bits(host_array(g.vc, "f32")), bits(vc))
        outs.append(og)
    # decode == last row of a one-shot prefill over the same 144 tokens (P3 §3.1), on the GPU
    q = np.concatenate([s.q for s in w.steps])
    full = W.Step(q=q, k_new=np.concatenate([s.k_new for s in w.steps]),
                  v_new=np.concatenate([s.v_new for s in w.steps]),
                  slot_mapping=np.concatenate([s.slot_mapping for s in w.steps]),
                  seq_lens=np.array([144], np.int32), query_start_loc=np.array([0, 144], np.int32),
                  block_tables=w.steps[0].block_tables)
    gf = GpuState(w)
    of = gf.step(full)
    for t in range(1, 17):
        assert np.max(np.abs(outs[t][0] - of[127 + t])) <= 1e-5
    assert np.max(np.abs(outs[0] - of[:128])) <= 1e-5


@pytest.mark.timeout(600)
def test_c2_decode_batch():
    w = W.config2()
    say("c2 generated")
    run_and_compare(w, what="c2")


@pytest.mark.timeout(600)
def test_c3_prefill_8k_sampled_rows():
    w = W.config3()
    rows = np.unique(np.concatenate([[0, 1, 2, 15, 16, 127, 128, 129, 255, 4095, 4096, 8190, 8191],
                                     np.random.default_rng(0).integers(0, 8192, 24)]))
    run_and_compare(w, rows=rows, what="c3 sampled rows")


@pytest.mark.timeout(600)
def test_c4_mixed_chunk():
    w = W.config4()
    st = w.steps[0]
    rng = np.random.default_rng(1)
    chunk_rows = 30 + np.unique(np.concatenate([[0, 1, 31, 32, 33, 1023, 2046, 2047], rng.integers(0, 2048, 16)]))
    rows = np.concatenate([np.arange(30), chunk_rows])
    out_g, _, _ = run_and_compare(w, rows=rows, what="c4 decodes + sampled chunk rows")


@pytest.mark.timeout(600)
def test_c5_skewed_long_decode():
    w = W.config5()
    run_and_compare(w, what="c5")


# ------------------------------------------------------------------------------------------
# invariants and probes on the GPU
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("chunks", [[1] * 20 + [300], [7, 7, 2, 304], [16, 17, 287], [128, 128, 64], [319, 1]])
def test_chunked_equals_one_shot(chunks):
    """P4 '把长输入切成块': chunked prefill gives the one-shot result (within rounding)."""
    S = sum(chunks)
    w = W.make_batch(77, [S], [S], 8, 2, 128, "bf16", num_blocks=24)
    one = GpuState(w).step(w.steps[0])
    cw = W.chunked_steps(w, chunks)
    g = GpuState(cw)
    c = 0
    for st in cw.steps:
        o = g.step(st)
        n = st.num_tokens
        compare(o, one[c:c + n], "bf16", what=f"chunk at {c}")
        c += n


def test_block_permutation_invariance_bitwise():
    lens, ql = [700, 47, 300], [1, 1, 130]
    a = W.make_batch(33, lens, ql, 8, 2, 128, "bf16", num_blocks=80, shuffle=False)
    b = W.make_batch(33, lens, ql, 8, 2, 128, "bf16", num_blocks=80, shuffle=True, rng=np.random.default_rng(9))
    sa, sb = a.steps[0], b.steps[0]
    kcb, vcb = W.poison_cache(b.k_cache0.shape, "bf16")
    for r in range(3):
        ctx = lens[r] - ql[r]
        pa_ = W.slots_for(sa.block_tables, r, np.arange(ctx))
        pb_ = W.slots_for(sb.block_tables, r, np.arange(ctx))
        kcb.reshape(-1, 2, 128)[pb_] = a.k_cache0.reshape(-1, 2, 128)[pa_]
        vcb.reshape(-1, 2, 128)[pb_] = a.v_cache0.reshape(-1, 2, 128)[pa_]
    stb = W.Step(q=sa.q, k_new=sa.k_new, v_new=sa.v_new, slot_mapping=sb.slot_mapping, seq_lens=sa.seq_lens,
                 query_start_loc=sa.query_start_loc, block_tables=sb.block_tables)
    oa = GpuState(a).step(sa)
    ob = GpuState(b, kcb, vcb).step(stb)
    assert np.array_equal(oa, ob)


def test_poison_has_no_effect_bitwise():
    """Unused blocks and tail slots hold NaN / +-3e38; replacing them with zeros changes no bit."""
    w = W.make_batch(4, [70, 33, 500], [3, 33, 1], 8, 2, 128, "bf16", num_blocks=60)
    st = w.steps[0]
    o_poison = GpuState(w).step(st)
    zk, zv = np.zeros_like(w.k_cache0), np.zeros_like(w.v_cache0)
    for b, s in enumerate(st.seq_lens):
        ctx = int(s) - int(st.q_lens[b])
        sl = W.slots_for(st.block_tables, b, np.arange(ctx))
        zk.reshape(-1, 2, 128)[sl] = w.k_cache0.reshape(-1, 2, 128)[sl]
        zv.reshape(-1, 2, 128)[sl] = w.v_cache0.reshape(-1, 2, 128)[sl]
    o_zero = GpuState(w, zk, zv).step(st)
    assert np.all(np.isfinite(W.to_float(o_poison, "bf16")))
    assert np.array_equal(o_poison, o_zero)


@pytest.mark.parametrize("dtype,prefill", [("f32", False), ("bf16", False), ("bf16", True)])
def test_argmax_probe_bit_exact(dtype, prefill):
    """q = 64 e0 and one key = 64 e0 (others 0): the target's weight rounds to exactly 1, so the
    output row equals that key's V row bit for bit -- through gather, splits and merge."""
    rng = np.random.default_rng(5)
    S, Hq, Hkv, d = 1100, 8, 2, 128
    for target in [0, 15, 16, 17, 255, 256, 511, 512, 777, S - 1]:
        q_len = 40 if prefill else 1
        w = W.make_batch(1, [S], [q_len], Hq, Hkv, d, dtype, num_blocks=80)
        st = w.steps[0]
        kf = np.zeros((S, Hkv, d), np.float32)
        kf[target, :, 0] = 64.0
        vf = rng.standard_normal((S, Hkv, d)).astype(np.float32)
        kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
        ctx = S - q_len
        slots = W.slots_for(st.block_tables, 0, np.arange(S))
        kc.reshape(-1, Hkv, d)[slots[:ctx]] = W.to_storage(kf[:ctx], dtype)
        vc.reshape(-1, Hkv, d)[slots[:ctx]] = W.to_storage(vf[:ctx], dtype)
        qf = np.zeros((q_len, Hq, d), np.float32)
        qf[:, :, 0] = 64.0
        st2 = W.Step(q=W.to_storage(qf, dtype), k_new=W.to_storage(kf[ctx:], dtype),
                     v_new=W.to_storage(vf[ctx:], dtype), slot_mapping=st.slot_mapping, seq_lens=st.seq_lens,
                     query_start_loc=st.query_start_loc, block_tables=st.block_tables)
        o = GpuState(w, kc, vc).step(st2)
        expect = np.repeat(W.to_storage(vf[target], dtype), Hq // Hkv, axis=0)
        for r in range(q_len):
            if ctx + r >= target:      # rows that can see the target
                assert np.array_equal(o[r], expect), (target, r)


def test_repeat_runs_are_bitwise_identical():
    w = W.make_batch(8, [900, 64, 3000], [1, 64, 1], 32, 8, 128, "bf16")
    g = GpuState(w)
    st = w.steps[0]
    o1 = g.step(st)
    o2 = g.step(st, append=False)
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------------------------------------
# check mode and host validation (nothing invalid ever reaches a data kernel)
# ------------------------------------------------------------------------------------------
def test_check_mode_reports_bad_block_id_and_bad_slot():
    w = W.make_batch(3, [40], [1], 2, 2, 128, "bf16", num_blocks=4)
    st = w.steps[0]
    g = GpuState(w)
    x = g.inputs(st)
    bt = st.block_tables.copy()
    bt[0, 1] = 99
    out = torch.empty_like(x["q"])
    with pytest.raises(pa.PAError) as e:
        pa.attention(x["q"], g.kc, g.vc, int_tensor(bt), x["sl"], x["qsl"], w.scale, out)
    assert e.value.code == 5 and "block id" in str(e.value)
    with pytest.raises(pa.PAError) as e:
        pa.append_kv(x["k"], x["v"], int_tensor(np.array([4 * 16], np.int32)), g.kc, g.vc)
    assert e.value.code == 5
    with pytest.raises(pa.PAError) as e:
        pa.attention(x["q"], g.kc, g.vc, x["bt"], int_tensor(np.array([4 * 16 + 1], np.int32)), x["qsl"], w.scale, out)
    assert e.value.code == 5


def test_binding_rejects_wrong_tensors():
    w = W.make_batch(3, [40], [1], 2, 2, 128, "bf16", num_blocks=4)
    g = GpuState(w)
    x = g.inputs(w.steps[0])
    out = torch.empty_like(x["q"])
    T, Hq, d = x["q"].shape
    q_strided = torch.zeros((T, Hq, 2 * d), dtype=x["q"].dtype, device=DEV)[..., :d]
    assert not q_strided.is_contiguous()
    with pytest.raises(ValueError):
        pa.attention(q_strided, g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out)
    with pytest.raises(TypeError):
        pa.attention(x["q"].float(), g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out)
    with pytest.raises(ValueError):
        pa.attention(x["q"].cpu(), g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out)
