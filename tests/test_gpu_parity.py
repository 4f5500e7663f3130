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
from tests.gpu_helpers import DEV, GpuState, compare, dev_tensor, host_array, int_tensor, say, tile_rows

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
def test_c3_prefill_8k_every_tile():
    """Every 256-row tile (all 32 KV heads, so every workgroup of the launch): its first and last
    rows, one row in each wave's slice, plus random rows."""
    w = W.config3()
    rows = tile_rows(0, 8192, 256 // (w.num_q_heads // w.num_kv_heads), np.random.default_rng(0), n_random=24)
    say(f"c3: {len(rows)} rows")
    run_and_compare(w, rows=rows, what="c3 rows of every tile")


@pytest.mark.timeout(600)
def test_c4_mixed_chunk_every_tile():
    """Every decode row and, for the chunk, every 64-position tile (first and last rows, a row per
    wave) plus random rows."""
    w = W.config4()
    rows = np.concatenate([np.arange(30), tile_rows(30, 2048, 256 // 4, np.random.default_rng(1))])
    say(f"c4: {len(rows)} rows")
    run_and_compare(w, rows=rows, what="c4 decodes + rows of every chunk tile")


def one_shot_of_last_request(w, rng):
    """The last request of a one-step workload as a one-shot prefill of its whole sequence: the
    cached context's K/V read back through its table, the step's own tokens appended after it; the
    query rows before the step's are fresh N(0,1) draws (their outputs are not compared)."""
    st = w.steps[0]
    b = st.num_seqs - 1
    s, ql = int(st.seq_lens[b]), int(st.q_lens[b])
    ctx, q0 = s - ql, int(st.query_start_loc[b])
    slots = W.slots_for(st.block_tables, b, np.arange(s))
    Hkv, d = w.num_kv_heads, w.head_dim
    k_all = np.concatenate([w.k_cache0.reshape(-1, Hkv, d)[slots[:ctx]], st.k_new[q0:q0 + ql]])
    v_all = np.concatenate([w.v_cache0.reshape(-1, Hkv, d)[slots[:ctx]], st.v_new[q0:q0 + ql]])
    q_all = np.concatenate([W.normal_storage(rng, (ctx, w.num_q_heads, d), w.dtype), st.q[q0:q0 + ql]])
    return W.Step(q=q_all, k_new=k_all, v_new=v_all, slot_mapping=slots.astype(np.int32),
                  seq_lens=np.array([s], np.int32), query_start_loc=np.array([0, s], np.int32),
                  block_tables=np.ascontiguousarray(st.block_tables[b:b + 1]))


@pytest.mark.timeout(600)
def test_c4_chunk_equals_one_shot_30720_prefill():
    """P4 '把长输入切成块': chunk 15 of the 30720-token prompt (2048 rows over 28672 cached keys, in
    the mixed step) gives the rows of a one-shot 30720-token prefill, both on the GPU.  The tiles of
    the two calls cover the same absolute positions and keys in the same order, so the rows agree
    bit for bit."""
    w = W.config4()
    st = w.steps[0]
    mixed = GpuState(w).step(st)
    one = one_shot_of_last_request(w, np.random.default_rng(44))
    full = GpuState(w).step(one)
    say("c4 chunk vs one-shot 30720: last 2048 rows")
    compare(mixed[30:], full[28672:], "bf16", what="c4 chunk vs one-shot")
    assert np.array_equal(mixed[30:], full[28672:])
@pytest.mark.timeout(600)
def test_c5_skewed_long_decode():
    w = W.config5()
    run_and_compare(w, what="c5")


# ------------------------------------------------------------------------------------------
# padding slots and the last blocks of the pool (64-bit offsets)
# ------------------------------------------------------------------------------------------
def relabel_blocks(w, top):
    """The same workload with physical blocks renamed so that its `top` highest-numbered used blocks
    become the last blocks of the pool (NB-1, NB-2, ...): a permutation of block ids applied to the
    caches, tables and slots alike (pure data movement)."""
    st = w.steps[0]
    NB = w.num_blocks
    used = np.unique(st.block_tables[st.block_tables >= 0])
    src = [int(x) for x in used[::-1][:top]]            # highest used ids
    dst = list(range(NB - 1, NB - 1 - len(src), -1))    # last ids of the pool
    perm = np.arange(NB, dtype=np.int64)                 # old id -> new id: disjoint swaps
    for a, b in zip([x for x in src if x not in dst], [x for x in dst if x not in src]):
        perm[a], perm[b] = b, a
    kc = np.empty_like(w.k_cache0)
    vc = np.empty_like(w.v_cache0)
    kc[perm] = w.k_cache0
    vc[perm] = w.v_cache0
    bt = np.where(st.block_tables >= 0, perm[np.maximum(st.block_tables, 0)], -1).astype(np.int32)
    sm = (perm[st.slot_mapping // 16] * 16 + st.slot_mapping % 16).astype(np.int32)
    st2 = W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new, slot_mapping=sm, seq_lens=st.seq_lens,
                 query_start_loc=st.query_start_loc, block_tables=bt)
    return W.Workload(name=w.name + "_relabelled", dtype=w.dtype, num_q_heads=w.num_q_heads,
                      num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, num_blocks=NB, scale=w.scale,
                      k_cache0=kc, v_cache0=vc, steps=[st2], seed=w.seed, kv_dtype=w.kv_dtype,
                      k_scale=w.k_scale, v_scale=w.v_scale)


def with_padding_tokens(w, every, rng):
    """The step's append gets a padding token (slot -1, random K/V) after every `every`-th token;
    the attention call is unchanged (P1 §2.2: rows are written at their page index, padding has
    none)."""
    st = w.steps[0]
    T = st.num_tokens
    pos = np.arange(0, T, every)
    n = len(pos)
    kpad = W.normal_storage(rng, (n,) + st.k_new.shape[1:], w.dtype)
    vpad = W.normal_storage(rng, (n,) + st.v_new.shape[1:], w.dtype)
    k = np.insert(st.k_new, pos + 1, kpad, axis=0)
    v = np.insert(st.v_new, pos + 1, vpad, axis=0)
    sm = np.insert(st.slot_mapping, pos + 1, -1).astype(np.int32)
    return k, v, sm


@pytest.mark.parametrize("kind", ["bf16_c2_pool", "f32_over_2GiB", "i8_over_2GiB"])
@pytest.mark.timeout(900)
def test_append_padding_and_last_pool_blocks(kind):
    """Padding tokens (slot < 0) are skipped and the pool's last blocks are written and read: caches
    compared byte for byte over the whole pool, attention against the oracle on every row.  The c2
    pool is exactly 2^31 bytes per cache; the other two pools exceed 2^31 bytes, so the last blocks'
    byte offsets need 64 bits."""
    rng = np.random.default_rng(71)
    if kind == "bf16_c2_pool":
        w = W.make_batch(71, [3000, 17, 1000, 256, 33], [1, 17, 1, 3, 1], 32, 32, 128, "bf16", num_blocks=16384,
                         max_blocks=256)
    elif kind == "f32_over_2GiB":
        w = W.make_batch(72, [700, 40, 129], [1, 40, 2], 16, 8, 64, "f32", num_blocks=66000)
    else:
        w = W.make_batch(73, [2000, 70, 513], [1, 70, 1], 64, 32, 128, "bf16", num_blocks=33000, cache="i8")
    cache_bytes = w.k_cache0.nbytes
    say(f"{kind}: cache {cache_bytes / 2**30:.3f} GiB, pool {w.num_blocks} blocks")
    w = relabel_blocks(w, top=4)
    st = w.steps[0]
    assert int(st.block_tables.max()) == w.num_blocks - 1
    k, v, sm = with_padding_tokens(w, 3, rng)
    g = GpuState(w)
    dt = w.dtype
    pa.append_kv(dev_tensor(k, dt), dev_tensor(v, dt), int_tensor(sm), g.kc, g.vc, g.ks, g.vs)
    x = g.inputs(st)
    out = torch.empty_like(x["q"])
    pa.attention(x["q"], g.kc, g.vc, x["bt"], x["sl"], x["qsl"], w.scale, out, k_scale=g.ks, v_scale=g.vs)
    torch.cuda.synchronize()
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    oracle.append(k, v, sm, kc, vc, w.k_scale, w.v_scale)
    ref, _ = oracle.attention(st.q, kc, vc, st.block_tables, st.seq_lens, st.query_start_loc, w.scale,
                              k_scale=w.k_scale, v_scale=w.v_scale)
    assert np.array_equal(bits(host_array(g.kc, w.cache_dtype)), bits(kc)), f"{kind}: K cache differs"
    assert np.array_equal(bits(host_array(g.vc, w.cache_dtype)), bits(vc)), f"{kind}: V cache differs"
    compare(host_array(out, dt), ref, dt, what=kind)


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


@pytest.mark.parametrize("d", [64, 128])
def test_two_and_four_head_decode_workgroups_agree_bitwise(d):
    """bf16 decode rows are served by workgroups of four KV heads, or of two (one wave per SIMD) on
    grids of at least two chip-wide rounds.  The same rows in a grid just under that size and, with
    one more row, just over it give identical outputs bit for bit: every wave computes its KV head
    the same way in both forms."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Hkv, splits = 8, 16                       # rows of up to 4096 keys: 16 splits of 256 keys
    over = -(-4 * cus // ((Hkv // 4) * splits))
    rng = np.random.default_rng(21)
    lens = rng.integers(3000, 4096, size=over, endpoint=True)
    w = W.make_batch(21, lens, np.ones(over, np.int64), 32, Hkv, d, "bf16", max_blocks=256)
    st = w.steps[0]
    n = over - 1
    st_under = W.Step(q=st.q[:n], k_new=st.k_new[:n], v_new=st.v_new[:n], slot_mapping=st.slot_mapping[:n],
                      seq_lens=st.seq_lens[:n], query_start_loc=st.query_start_loc[:n + 1],
                      block_tables=st.block_tables[:n])
    o_over = GpuState(w).step(st)
    o_under = GpuState(w).step(st_under)
    say(f"  d = {d}: {over} rows (two-head workgroups) against {n} (four-head workgroups)")
    assert np.array_equal(o_over[:n], o_under)
    compare(o_over, oracle_out(w, st, w.k_cache0.copy(), w.v_cache0.copy(), rows=[0, n // 2, n]), "bf16",
            rows=[0, n // 2, n], what="two-head workgroups")


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
