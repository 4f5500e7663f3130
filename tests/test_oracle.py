"""Pins for the CPU oracle: things the pages and the mathematics fix, independent of the oracle.

Sources: P1 "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576); P3 prefill/decode article on
the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127); P4 "11. 分块预填充与统一调度"
(niuwancheng.cn, llm-inference/11-chunked-prefill).
"""
import math

import numpy as np
import pytest
import torch

from attention_paged_kv_amd import workloads as W
import oracle
from tests.oracle_helpers import logical_kv, oracle_step

TOL64 = 1e-12


def sdpa_dense(q, k, v, scale):
    """Library dense causal softmax (torch CPU, float64) on contiguous [S, H, d] inputs.

    GQA is expressed as MHA with each KV head repeated for its contiguous group of query heads."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0).unsqueeze(0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.squeeze(0).permute(1, 0, 2).numpy()


def f64(w, a):
    return W.to_float(a, w.dtype).astype(np.float64)


# --------------------------------------------------------------------------------------------
# 1. Dense causal softmax from a library routine, tiny inputs (P3 §2.1: the upper triangle is
#    masked to -inf before the row softmax, then the weights multiply V).
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("S,Hq,Hkv,d,dtype,shuffle", [
    (1, 1, 1, 64, "f32", False),
    (15, 2, 2, 64, "f32", True),
    (16, 4, 4, 64, "f32", True),
    (17, 4, 1, 64, "f32", True),
    (33, 8, 2, 128, "bf16", True),
    (100, 4, 4, 64, "bf16", False),
    (257, 6, 3, 64, "f32", True),
])
def test_prefill_matches_library_dense_causal_softmax(S, Hq, Hkv, d, dtype, shuffle):
    w = W.make_batch(11 + S, [S], [S], Hq, Hkv, d, dtype, num_blocks=(S + 15) // 16 + 3, shuffle=shuffle)
    st = w.steps[0]
    _, o64, _, _ = oracle_step(w)
    ref = sdpa_dense(f64(w, st.q), f64(w, st.k_new), f64(w, st.v_new), w.scale)
    assert np.max(np.abs(o64 - ref)) <= TOL64


def test_multi_request_prefill_matches_library():
    """Several requests in one varlen batch, each checked against its own dense softmax."""
    lens = [1, 15, 16, 17, 31, 32, 33, 64]
    w = W.make_batch(5, lens, lens, 4, 2, 64, "bf16", num_blocks=sum((s + 15) // 16 for s in lens) + 5)
    st = w.steps[0]
    _, o64, _, _ = oracle_step(w)
    for b in range(len(lens)):
        a, e = st.query_start_loc[b], st.query_start_loc[b + 1]
        ref = sdpa_dense(f64(w, st.q[a:e]), f64(w, st.k_new[a:e]), f64(w, st.v_new[a:e]), w.scale)
        assert np.max(np.abs(o64[a:e] - ref)) <= TOL64, b


# --------------------------------------------------------------------------------------------
# 2. Page invariants.
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("chunks", [[1] * 40, [7] * 5 + [5], [16, 17, 7], [2, 38], [39, 1], [13, 13, 14]])
def test_chunked_prefill_equals_one_shot(chunks):
    """P4 '把长输入切成块': a chunk reads the cached KV of earlier chunks, then writes its own; the
    result is the same as computing the whole prompt at once."""
    S = sum(chunks)
    w = W.make_batch(21, [S], [S], 4, 2, 64, "bf16", num_blocks=8)
    _, one64, _, _ = oracle_step(w)
    cw = W.chunked_steps(w, chunks)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    c = 0
    for st in cw.steps:
        _, o64 = oracle.run_step(cw, st, kc, vc, want_f64=True)
        n = st.num_tokens
        assert np.max(np.abs(o64 - one64[c:c + n])) <= TOL64
        c += n


def test_decode_steps_equal_last_rows_of_full_prefill():
    """P3 §3.1: a decode step appends the new token's K/V and attends over all S+t keys, so it must
    equal the matching row of a one-shot prefill over the same tokens (config c1 shapes)."""
    w = W.config1()
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    outs = []
    for st in w.steps:
        o, _ = oracle.run_step(w, st, kc, vc)
        outs.append(o)
    # one-shot prefill of all 144 tokens with the same table
    q = np.concatenate([s.q for s in w.steps])
    kn = np.concatenate([s.k_new for s in w.steps])
    vn = np.concatenate([s.v_new for s in w.steps])
    sm = np.concatenate([s.slot_mapping for s in w.steps])
    full = W.Step(q=q, k_new=kn, v_new=vn, slot_mapping=sm, seq_lens=np.array([144], np.int32),
                  query_start_loc=np.array([0, 144], np.int32), block_tables=w.steps[0].block_tables)
    of, _ = oracle.run_step(w, full, w.k_cache0.copy(), w.v_cache0.copy())
    assert np.array_equal(outs[0], of[:128])
    for t in range(1, 17):
        assert np.array_equal(outs[t][0], of[127 + t]), t


# --------------------------------------------------------------------------------------------
# 3. Closed forms.
# --------------------------------------------------------------------------------------------
def _prefill(S, Hq, Hkv, d, dtype="f32", seed=3):
    return W.make_batch(seed, [S], [S], Hq, Hkv, d, dtype, num_blocks=(S + 15) // 16 + 1)


def _with_new_kv(w, k_new=None, v_new=None):
    st = w.steps[0]
    st2 = W.Step(q=st.q, k_new=st.k_new if k_new is None else k_new, v_new=st.v_new if v_new is None else v_new,
                 slot_mapping=st.slot_mapping, seq_lens=st.seq_lens, query_start_loc=st.query_start_loc,
                 block_tables=st.block_tables)
    return st2


def test_constant_values_give_that_constant():
    """If every V row equals c, any convex combination of them is c."""
    w = _prefill(50, 4, 2, 64)
    c = np.random.default_rng(0).standard_normal((1, 2, 64)).astype(np.float32)
    st = _with_new_kv(w, v_new=np.repeat(c, 50, axis=0))
    _, o64, _, _ = oracle_step(w, st)
    expect = np.repeat(c.astype(np.float64), 2, axis=1)  # q-head h uses KV head h // 2
    assert np.max(np.abs(o64 - expect[None, 0])) <= 1e-14


@pytest.mark.parametrize("zero", ["k", "scale"])
def test_flat_scores_give_prefix_mean(zero):
    """With all scores equal (K = 0, or scale = 0) the softmax is uniform over the visible keys,
    so row r is the mean of V[0..r]."""
    w = _prefill(40, 2, 2, 64)
    st = w.steps[0]
    if zero == "k":
        st = _with_new_kv(w, k_new=np.zeros_like(st.k_new))
    else:
        w.scale = 0.0
    _, o64, _, _ = oracle_step(w, st)
    v = st.v_new.astype(np.float64)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, 41)[:, None, None]
    assert np.max(np.abs(o64 - prefix_mean)) <= 1e-13


def test_first_prefill_row_is_first_value_exactly():
    """Row 0 of a prefill from position 0 sees a single key, so its output is V[0] exactly."""
    for dtype in ("f32", "bf16"):
        w = _prefill(20, 4, 4, 64, dtype)
        out, _, _, _ = oracle_step(w)
        assert np.array_equal(out[0], w.steps[0].v_new[0])


def test_gqa_equals_mha_with_repeated_kv_heads():
    """Grouped-query attention (P3 §2.3: fewer KV heads serve the query heads) equals multi-head
    attention where each KV head is repeated for its contiguous group of query heads."""
    w = W.make_batch(9, [37, 5, 70], [37, 1, 9], 8, 2, 64, "bf16", num_blocks=12)
    out_g, _, _, _ = oracle_step(w)
    rep = lambda a: np.ascontiguousarray(np.repeat(a, 4, axis=-2))
    st = w.steps[0]
    wm = W.Workload(name="mha", dtype=w.dtype, num_q_heads=8, num_kv_heads=8, head_dim=64, num_blocks=w.num_blocks,
                    scale=w.scale, k_cache0=rep(w.k_cache0), v_cache0=rep(w.v_cache0))
    stm = W.Step(q=st.q, k_new=rep(st.k_new), v_new=rep(st.v_new), slot_mapping=st.slot_mapping,
                 seq_lens=st.seq_lens, query_start_loc=st.query_start_loc, block_tables=st.block_tables)
    out_m, _, _, _ = oracle_step(wm, stm)
    assert np.array_equal(out_g, out_m)


# --------------------------------------------------------------------------------------------
# 4. Indexing: argmax probes, block-permutation invariance, poison invariance.
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_probe_returns_target_value_bit_exactly(dtype):
    rng = np.random.default_rng(7)
    d, Hq, Hkv = 128, 4, 2
    S = 67
    for target in [0, 14, 15, 16, 17, 40, S - 1, int(rng.integers(0, S))]:
        w = W.make_batch(1, [S], [1], Hq, Hkv, d, dtype)
        st = w.steps[0]
        kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
        NB = kc.shape[0]
        kf = np.zeros((S, Hkv, d), np.float32)
        kf[target, :, 0] = 64.0
        vf = rng.standard_normal((S, Hkv, d)).astype(np.float32)
        slots = W.slots_for(st.block_tables, 0, np.arange(S))
        kc.reshape(NB * 16, Hkv, d)[slots[:-1]] = W.to_storage(kf[:-1], dtype)
        vc.reshape(NB * 16, Hkv, d)[slots[:-1]] = W.to_storage(vf[:-1], dtype)
        qf = np.zeros((1, Hq, d), np.float32)
        qf[:, :, 0] = 64.0
        st2 = W.Step(q=W.to_storage(qf, dtype), k_new=W.to_storage(kf[-1:], dtype), v_new=W.to_storage(vf[-1:], dtype),
                     slot_mapping=st.slot_mapping, seq_lens=st.seq_lens, query_start_loc=st.query_start_loc,
                     block_tables=st.block_tables)
        out, _, _, _ = oracle_step(w, st2, caches=(kc, vc))
        expect = np.repeat(W.to_storage(vf[target], dtype), Hq // Hkv, axis=0)  # head h -> KV head h // G
        assert np.array_equal(out[0], expect), target


def test_dominant_future_key_is_masked():
    """A huge score at a position after the query (chunk rows before the end) must not leak in:
    rows before that position equal those computed without it."""
    w = W.make_batch(2, [60], [60], 2, 2, 64, "f32")
    st = w.steps[0]
    out0, _, _, _ = oracle_step(w)
    k2 = st.k_new.copy()
    k2[45] = 1e3 * st.q[0, 0][None]
    out1, _, _, _ = oracle_step(w, _with_new_kv(w, k_new=k2))
    assert np.array_equal(out0[:45], out1[:45])
    assert not np.array_equal(out0[45:], out1[45:])


def test_block_permutation_invariance_bitwise():
    """Only the physical placement differs -> identical output bits."""
    lens, ql = [300, 47, 128], [300, 1, 20]
    a = W.make_batch(33, lens, ql, 4, 2, 64, "bf16", num_blocks=40, shuffle=False)
    b = W.make_batch(33, lens, ql, 4, 2, 64, "bf16", num_blocks=40, shuffle=True,
                     rng=np.random.default_rng(1234))
    # same values, different placement: rebuild b's values from a's logical content
    sa, sb = a.steps[0], b.steps[0]
    kcb, vcb = W.poison_cache(b.k_cache0.shape, "bf16")
    kca, vca = a.k_cache0, a.v_cache0
    for r in range(3):
        ctx = lens[r] - ql[r]
        pa_ = W.slots_for(sa.block_tables, r, np.arange(ctx))
        pb_ = W.slots_for(sb.block_tables, r, np.arange(ctx))
        kcb.reshape(-1, 2, 64)[pb_] = kca.reshape(-1, 2, 64)[pa_]
        vcb.reshape(-1, 2, 64)[pb_] = vca.reshape(-1, 2, 64)[pa_]
    stb = W.Step(q=sa.q, k_new=sa.k_new, v_new=sa.v_new, slot_mapping=sb.slot_mapping, seq_lens=sa.seq_lens,
                 query_start_loc=sa.query_start_loc, block_tables=sb.block_tables)
    oa, _, _, _ = oracle_step(a)
    ob, _, _, _ = oracle_step(b, stb, caches=(kcb, vcb))
    assert not np.array_equal(sa.block_tables, sb.block_tables)
    assert np.array_equal(oa, ob)


def test_poison_outside_visible_range_has_no_effect():
    w = W.make_batch(4, [70, 33], [3, 33], 4, 4, 64, "bf16", num_blocks=20)
    out_p, _, _, _ = oracle_step(w)
    assert np.all(np.isfinite(W.to_float(out_p, "bf16")))
    zk = np.zeros_like(w.k_cache0)
    zv = np.zeros_like(w.v_cache0)
    st = w.steps[0]
    for b, s in enumerate(st.seq_lens):
        ctx = int(s) - int(st.q_lens[b])
        sl = W.slots_for(st.block_tables, b, np.arange(ctx))
        zk.reshape(-1, 4, 64)[sl] = w.k_cache0.reshape(-1, 4, 64)[sl]
        zv.reshape(-1, 4, 64)[sl] = w.v_cache0.reshape(-1, 4, 64)[sl]
    out_z, _, _, _ = oracle_step(w, caches=(zk, zv))
    assert np.array_equal(out_p, out_z)


# --------------------------------------------------------------------------------------------
# 5. Append (P3 §2.3 only K and V are cached; P1 §2.2 each token is written at its page slot).
# --------------------------------------------------------------------------------------------
def test_append_writes_rows_at_slots_and_nothing_else():
    w = W.make_batch(8, [40, 17], [40, 2], 2, 2, 64, "bf16", num_blocks=8)
    st = w.steps[0]
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    oracle.append(st.k_new, st.v_new, st.slot_mapping, kc, vc)
    flat_k, flat_v = kc.reshape(-1, 2, 64), vc.reshape(-1, 2, 64)
    assert np.array_equal(flat_k[st.slot_mapping], st.k_new)
    assert np.array_equal(flat_v[st.slot_mapping], st.v_new)
    untouched = np.ones(flat_k.shape[0], bool)
    untouched[st.slot_mapping] = False
    assert np.array_equal(flat_k[untouched], w.k_cache0.reshape(-1, 2, 64)[untouched])
    assert np.array_equal(flat_v[untouched], w.v_cache0.reshape(-1, 2, 64)[untouched])


def test_append_skips_negative_slots_and_rejects_bad_ones():
    kc, vc = W.poison_cache((2, 16, 1, 64), "f32")
    k = np.ones((3, 1, 64), np.float32)
    before = kc.copy()
    oracle.append(k, k, np.array([-1, -5, -1], np.int32), kc, vc)
    assert np.array_equal(kc, before)
    with pytest.raises(oracle.OracleError):
        oracle.append(k, k, np.array([0, 32, 1], np.int32), kc, vc)
    with pytest.raises(oracle.OracleError):
        oracle.append(k, k, np.array([3, 4, 3], np.int32), kc, vc)


def test_attention_rejects_bad_descriptors():
    w = W.make_batch(8, [20], [4], 2, 2, 64, "f32", num_blocks=3)
    st = w.steps[0]
    with pytest.raises(oracle.OracleError):   # q_len > seq_len
        oracle.attention(st.q, w.k_cache0, w.v_cache0, st.block_tables, np.array([3], np.int32),
                         st.query_start_loc, w.scale)
    bt = st.block_tables.copy()
    bt[0, 1] = 99
    with pytest.raises(oracle.OracleError):   # block outside the pool
        oracle.attention(st.q, w.k_cache0, w.v_cache0, bt, st.seq_lens, st.query_start_loc, w.scale)


# --------------------------------------------------------------------------------------------
# 6. Output rounding to bf16 (nearest, ties to even, one rounding from the exact value).
# --------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_library_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-40, 38, 2000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0, 3.3e38, 1e-40,
                                  -1e-42, 0.0, -0.0], np.float32)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.f64_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(mine, lib)


def test_bf16_rounding_is_single_step_from_double():
    # exact tie -> even; just above the tie (only visible in double) -> up; overflow -> inf
    assert oracle.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    assert oracle.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert oracle.f64_to_bf16(-(1.0 + 2 ** -8 + 2 ** -40)) == 0xBF81
    assert oracle.f64_to_bf16(3.4e38) == 0x7F80
    assert oracle.f64_to_bf16(float("nan")) == 0x7FC0
    assert oracle.f64_to_bf16(2.0 ** -133) == 0x0001
    assert oracle.f64_to_bf16(2.0 ** -134) == 0x0000          # tie at half the smallest subnormal -> even (0)
    assert oracle.f64_to_bf16(2.0 ** -134 * 1.0000001) == 0x0001


# --------------------------------------------------------------------------------------------
# 7. Sliding window (P2 §5.2 and P3 §6.3: only the most recent W tokens' K/V take part).  Reading:
#    the query at position p sees keys p - W + 1 .. p, itself included; W = 0 means no window.
# --------------------------------------------------------------------------------------------
def _sdpa_rows_over_windows(q, k, v, scale, ctx, window):
    """Library softmax(q K^T) V per query row over the contiguous slice of keys its window covers."""
    Hq, Hkv = q.shape[1], k.shape[1]
    out = np.empty_like(q)
    for r in range(q.shape[0]):
        p = ctx + r
        lo = max(0, p - window + 1)
        qt = torch.from_numpy(q[r:r + 1]).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(k[lo:p + 1]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0).unsqueeze(0)
        vt = torch.from_numpy(v[lo:p + 1]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0).unsqueeze(0)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        out[r] = o.squeeze(0).permute(1, 0, 2).numpy()[0]
    return out


@pytest.mark.parametrize("lens,qlens,window", [
    ([70], [70], 1), ([70], [70], 16), ([70], [70], 17), ([100, 33, 64], [100, 1, 9], 31),
    ([300, 47], [5, 1], 64), ([40], [40], 39),
])
def test_window_matches_library_softmax_over_each_rows_window(lens, qlens, window):
    w = W.make_batch(40 + window, lens, qlens, 4, 2, 64, "bf16",
                     num_blocks=sum((s + 15) // 16 for s in lens) + 4)
    st = w.steps[0]
    _, o64, kc, vc = oracle_step(w, window=window)
    for b in range(len(lens)):
        a, e = st.query_start_loc[b], st.query_start_loc[b + 1]
        k, v = logical_kv(w, st, kc, vc, b)
        ref = _sdpa_rows_over_windows(f64(w, st.q[a:e]), k, v, w.scale, int(st.seq_lens[b]) - (e - a), window)
        assert np.max(np.abs(o64[a:e] - ref)) <= TOL64, b


@pytest.mark.parametrize("window", [100, 101, 5000])
def test_window_at_least_the_context_is_full_causal_bitwise(window):
    w = W.make_batch(8, [100, 40], [100, 3], 4, 2, 64, "bf16", num_blocks=12)
    full, _, _, _ = oracle_step(w)
    win, _, _, _ = oracle_step(w, window=window)
    assert np.array_equal(full, win)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_one_returns_own_value_exactly(dtype):
    """With W = 1 each row sees only its own key, so the output is its own V row."""
    w = W.make_batch(9, [50, 20], [50, 4], 4, 4, 64, dtype, num_blocks=10)
    st = w.steps[0]
    out, _, _, _ = oracle_step(w, window=1)
    assert np.array_equal(out, st.v_new)


def test_window_chunked_equals_one_shot_and_decode_equals_last_row():
    S, Wn = 90, 23
    w = W.make_batch(12, [S], [S], 4, 2, 64, "bf16", num_blocks=8)
    one, _, _, _ = oracle_step(w, window=Wn)
    cw = W.chunked_steps(w, [30, 17, 1, 1, 41])
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    c = 0
    for st in cw.steps:
        o, _ = oracle.run_step(cw, st, kc, vc, window=Wn)
        n = o.shape[0]
        assert np.array_equal(o, one[c:c + n]), c
        c += n


def test_key_just_outside_window_is_masked_and_edge_key_is_not():
    """A dominant key at position p - W (one step too old) has no effect on row p; at p - W + 1
    it takes the whole softmax weight."""
    S, Wn, d = 64, 20, 64
    w = W.make_batch(3, [S], [1], 2, 2, d, "f32", num_blocks=6)
    st = w.steps[0]
    base, _, _, _ = oracle_step(w, window=Wn)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    NB = kc.shape[0]
    p = S - 1
    for pos, inside in [(p - Wn, False), (p - Wn + 1, True)]:
        k2, v2 = kc.copy(), vc.copy()
        slot = W.slots_for(st.block_tables, 0, np.array([pos]))[0]
        k2.reshape(NB * 16, 2, d)[slot] = 1e3 * st.q[0]
        out, _, _, _ = oracle_step(w, caches=(k2, v2), window=Wn)
        if inside:
            assert np.array_equal(out[0], v2.reshape(NB * 16, 2, d)[slot])
        else:
            assert np.array_equal(out[0], base[0])


def test_window_poison_and_unmapped_blocks_before_the_window_are_never_read():
    """Blocks wholly before the first row's window may hold anything, and their table entries may be
    outside the pool (a cache that drops old blocks); the output is unchanged."""
    lens, ql, Wn = [200, 97], [3, 1], 40
    w = W.make_batch(6, lens, ql, 4, 2, 64, "bf16", num_blocks=24)
    st = w.steps[0]
    ref, _, _, _ = oracle_step(w, window=Wn)
    kp, vp = W.poison_cache(w.k_cache0.shape, "bf16")
    tables = st.block_tables.copy()
    for b in range(2):
        s, q = lens[b], ql[b]
        lo = s - q - Wn + 1
        keep = np.arange(max(0, lo), s - q)
        sl = W.slots_for(st.block_tables, b, keep)
        kp.reshape(-1, 2, 64)[sl] = w.k_cache0.reshape(-1, 2, 64)[sl]
        vp.reshape(-1, 2, 64)[sl] = w.v_cache0.reshape(-1, 2, 64)[sl]
        tables[b, :max(0, lo) // 16] = -1
    st2 = W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new, slot_mapping=st.slot_mapping, seq_lens=st.seq_lens,
                 query_start_loc=st.query_start_loc, block_tables=tables)
    out, _, _, _ = oracle_step(w, st2, caches=(kp, vp), window=Wn)
    assert np.array_equal(out, ref)


def test_window_rejects_negative():
    w = W.make_batch(1, [20], [20], 2, 2, 64, "f32", num_blocks=3)
    with pytest.raises(Exception):
        oracle_step(w, window=-1)


# --------------------------------------------------------------------------------------------
# 8. 8-bit cache (P2 §4.3, §5.4: INT8 KV cache calibrated per channel).  Reading: symmetric codes
#    in [-127, 127], one fp32 scale per (KV head, channel); append rounds x / s, computed in fp32,
#    to the nearest integer with ties to even; NaN -> 0; attention reads code * s.
# --------------------------------------------------------------------------------------------
def test_quantize_closed_forms():
    s = 0.25
    for n in list(range(-127, 128, 7)) + [-127, 127, 0]:
        assert oracle.quantize(n * s, s) == n
    for n, even in [(0, 0), (1, 2), (2, 2), (-1, 0), (-2, -2), (-3, -2), (126, 126), (125, 126)]:
        assert oracle.quantize((n + 0.5) * s, s) == even, n         # ties go to the even code
    assert oracle.quantize(128 * s, s) == 127 and oracle.quantize(-1e30, s) == -127
    assert oracle.quantize(float("inf"), s) == 127 and oracle.quantize(float("-inf"), s) == -127
    assert oracle.quantize(float("nan"), s) == 0


def test_quantize_decides_in_single_precision():
    """The rounding follows the fp32 quotient (the library's IEEE division), also where the exact
    quotient lies on the other side of a half-integer."""
    rng = np.random.default_rng(0)
    disagreements = 0
    for _ in range(4000):
        sc = np.float32(rng.uniform(0.01, 0.05))
        n = int(rng.integers(-120, 120))
        x = np.float32((n + 0.5) * float(sc))
        q32 = np.float32(x) / np.float32(sc)
        expect = int(np.clip(np.rint(q32), -127, 127))
        assert oracle.quantize(float(x), float(sc)) == expect
        if expect != int(np.clip(np.rint(float(x) / float(sc)), -127, 127)):
            disagreements += 1
    assert disagreements > 0      # the sample exercises cases where fp64 would decide differently


def _i8_batch(seed, lens, qlens, Hq=4, Hkv=2, d=64, pow2=False):
    w = W.make_batch(seed, lens, qlens, Hq, Hkv, d, "bf16", num_blocks=sum((s + 15) // 16 for s in lens) + 3,
                     cache="i8")
    if pow2:
        rng = np.random.default_rng(seed)
        w.k_scale = (2.0 ** -rng.integers(4, 8, (Hkv, d))).astype(np.float32)
        w.v_scale = (2.0 ** -rng.integers(4, 8, (Hkv, d))).astype(np.float32)
    return w


def test_int8_append_writes_quantised_rows_at_slots_and_nothing_else():
    w = _i8_batch(31, [40, 20], [40, 3])
    st = w.steps[0]
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    oracle.append(st.k_new, st.v_new, st.slot_mapping, kc, vc, w.k_scale, w.v_scale)
    for new, cache0, cache, sc in [(st.k_new, w.k_cache0, kc, w.k_scale), (st.v_new, w.v_cache0, vc, w.v_scale)]:
        x = W.to_float(new, "bf16")
        expect = np.clip(np.rint(x / sc[None]), -127, 127).astype(np.int8)     # numpy fp32 division
        flat, flat0 = cache.reshape(-1, 2, 64), cache0.reshape(-1, 2, 64)
        assert np.array_equal(flat[st.slot_mapping], expect)
        others = np.setdiff1d(np.arange(flat.shape[0]), st.slot_mapping)
        assert np.array_equal(flat[others], flat0[others])


def test_int8_attention_equals_fp32_attention_over_dequantised_cache_bitwise():
    """With power-of-two scales every code * scale is exact in fp32, so reading the int8 cache must
    give the very doubles that the fp32 path computes from the dequantised cache."""
    w = _i8_batch(32, [300, 47, 128], [1, 1, 20], Hq=8, Hkv=2, d=64, pow2=True)
    st = w.steps[0]
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    _, o8 = oracle.run_step(w, st, kc, vc, want_f64=True)
    kf = (kc.astype(np.float32) * w.k_scale[None, None]).astype(np.float32)
    vf = (vc.astype(np.float32) * w.v_scale[None, None]).astype(np.float32)
    qf = W.to_float(st.q, "bf16")
    _, of = oracle.attention(qf, kf, vf, st.block_tables, st.seq_lens, st.query_start_loc, w.scale, want_f64=True)
    assert np.array_equal(o8, of)


@pytest.mark.parametrize("window", [0, 37])
def test_int8_attention_matches_library_softmax_over_dequantised_values(window):
    w = _i8_batch(33, [200, 65, 90], [1, 65, 7], Hq=4, Hkv=2, d=64)
    st = w.steps[0]
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    _, o64 = oracle.run_step(w, st, kc, vc, want_f64=True, window=window)
    for b in range(3):
        s = int(st.seq_lens[b])
        sl = W.slots_for(st.block_tables, b, np.arange(s))
        k = kc.reshape(-1, 2, 64)[sl].astype(np.float64) * w.k_scale[None].astype(np.float64)
        v = vc.reshape(-1, 2, 64)[sl].astype(np.float64) * w.v_scale[None].astype(np.float64)
        a, e = st.query_start_loc[b], st.query_start_loc[b + 1]
        ctx = s - (e - a)
        ref = _sdpa_rows_over_windows(f64(w, st.q[a:e]), k, v, w.scale, ctx, window or s)
        assert np.max(np.abs(o64[a:e] - ref)) <= TOL64, b


def test_int8_argmax_probe_returns_dequantised_target_exactly():
    d, Hq, Hkv, S = 64, 4, 2, 67
    for target in [0, 15, 16, 40, S - 1]:
        w = _i8_batch(34, [S], [1], Hq=Hq, Hkv=Hkv, d=d, pow2=True)
        w.k_scale[:, 0] = 1.0
        st = w.steps[0]
        kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
        slots = W.slots_for(st.block_tables, 0, np.arange(S))
        kflat = kc.reshape(-1, Hkv, d)
        kflat[slots[:-1]] = 0
        knew = np.zeros((1, Hkv, d), np.float32)
        if target == S - 1:
            knew[0, :, 0] = 127.0
        else:
            kflat[slots[target], :, 0] = 127
        qf = np.zeros((1, Hq, d), np.float32)
        qf[:, :, 0] = 64.0
        st2 = W.Step(q=W.to_storage(qf, "bf16"), k_new=W.to_storage(knew, "bf16"), v_new=st.v_new,
                     slot_mapping=st.slot_mapping, seq_lens=st.seq_lens, query_start_loc=st.query_start_loc,
                     block_tables=st.block_tables)
        out, _ = oracle.run_step(w, st2, kc, vc)
        vt = vc.reshape(-1, Hkv, d)[slots[target]].astype(np.float32) * w.v_scale      # exact
        expect = np.repeat(W.to_storage(vt, "bf16"), Hq // Hkv, axis=0)
        assert np.array_equal(out[0], expect), target
