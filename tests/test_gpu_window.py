"""GPU parity of sliding-window attention (P2 §5.2, P3 §6.3: only the most recent W tokens' K/V
take part; the row at position p sees keys p - W + 1 .. p) against the CPU oracle with the same
window.  Tolerances as for full causal attention; invariances are bitwise."""
import numpy as np
import pytest

import attention_paged_kv_amd as pa
from attention_paged_kv_amd import workloads as W
import oracle
from tests.gpu_helpers import GpuState, compare, host_array, say, tile_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def check_mode():
    pa.set_check(True)
    yield
    pa.set_check(False)


def run_window(w, window, rows=None, what=""):
    st = w.steps[0]
    g = GpuState(w)
    out_g = g.step(st, window=window)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    out_r, _ = oracle.run_step(w, st, kc, vc, rows=rows, window=window)
    compare(out_g, out_r, w.dtype, rows=rows, what=what)
    return out_g


CASES = [
    # seq_lens, q_lens, Hq, Hkv, d, dtype, window
    ([300, 33, 16], [1, 1, 1], 4, 4, 128, "f32", 17),
    ([70, 129, 5], [70, 2, 5], 4, 2, 64, "f32", 16),
    ([15, 16, 17, 31, 32, 33, 700], [1, 1, 1, 1, 1, 1, 1], 8, 2, 128, "bf16", 1),
    ([15, 16, 17, 31, 32, 33, 700], [1, 1, 1, 1, 1, 1, 1], 8, 2, 128, "bf16", 16),
    ([15, 16, 17, 31, 32, 33, 700], [1, 1, 1, 1, 1, 1, 1], 8, 2, 128, "bf16", 17),
    ([2000, 1300, 513], [1, 1, 1], 32, 8, 128, "bf16", 300),      # several splits after the window start
    ([2000, 1300, 513], [1, 1, 1], 32, 8, 128, "bf16", 1000),
    ([255, 256, 257], [255, 256, 257], 4, 4, 128, "bf16", 64),     # prefill tiles, window = one key tile
    ([255, 256, 257], [255, 256, 257], 4, 4, 128, "bf16", 65),
    ([400, 129], [129, 129], 16, 1, 64, "bf16", 100),
    ([1000, 513, 700], [1, 200, 64], 32, 8, 128, "bf16", 128),
    ([600, 300], [600, 300], 8, 8, 128, "bf16", 1),                # every row sees only itself
    ([1030, 1030], [1, 7], 32, 32, 128, "bf16", 250),
    ([900], [300], 8, 1, 128, "bf16", 37),                         # chunk: its window starts in the cache
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_window_small_batches(case):
    seq, ql, Hq, Hkv, d, dt, win = CASES[case]
    say(f"window case {case}: seq {seq} q {ql} Hq {Hq} Hkv {Hkv} d {d} {dt} W {win}")
    nb = sum((s + 15) // 16 for s in seq) + 3
    w = W.make_batch(500 + case, seq, ql, Hq, Hkv, d, dt, num_blocks=nb)
    run_window(w, win, what=f"window[{case}]")


@pytest.mark.parametrize("window", [700, 5000])
def test_window_covering_the_context_equals_no_window_bitwise(window):
    w = W.make_batch(41, [700, 47, 300], [1, 1, 130], 8, 2, 128, "bf16", num_blocks=80)
    st = w.steps[0]
    full = GpuState(w).step(st)
    win = GpuState(w).step(st, window=window)
    assert np.array_equal(full, win)


def test_window_ignores_poison_and_unmapped_blocks_before_it_bitwise():
    """Slots before each request's first window hold NaN / +-3e38 and the table entries of blocks
    wholly before it are -1 (a cache that dropped them); check mode accepts the call and the output
    equals the one computed with those slots zeroed and the entries valid."""
    lens, ql, win = [900, 97, 600, 1300], [3, 1, 200, 1], 160
    w = W.make_batch(6, lens, ql, 8, 2, 128, "bf16", num_blocks=200)
    st = w.steps[0]
    zk, zv = np.zeros_like(w.k_cache0), np.zeros_like(w.v_cache0)
    kp, vp = W.poison_cache(w.k_cache0.shape, "bf16")
    tables = st.block_tables.copy()
    for b in range(len(lens)):
        s, q = lens[b], ql[b]
        lo = max(0, s - q - win + 1)
        keep = W.slots_for(st.block_tables, b, np.arange(lo, s - q))
        for dst in (zk, kp):
            dst.reshape(-1, 2, 128)[keep] = w.k_cache0.reshape(-1, 2, 128)[keep]
        for dst in (zv, vp):
            dst.reshape(-1, 2, 128)[keep] = w.v_cache0.reshape(-1, 2, 128)[keep]
        tables[b, :lo // 16] = -1
    st_cut = W.Step(q=st.q, k_new=st.k_new, v_new=st.v_new, slot_mapping=st.slot_mapping, seq_lens=st.seq_lens,
                    query_start_loc=st.query_start_loc, block_tables=tables)
    o_zero = GpuState(w, zk, zv).step(st, window=win)
    o_poison = GpuState(w, kp, vp).step(st_cut, window=win)
    assert np.all(np.isfinite(W.to_float(o_poison, "bf16")))
    assert np.array_equal(o_poison, o_zero)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    out_r, _ = oracle.run_step(w, st, kc, vc, window=win)
    compare(o_poison, out_r, "bf16", what="poisoned window")


@pytest.mark.parametrize("chunks", [[100, 100, 120], [1] * 10 + [310], [64, 1, 255]])
def test_window_chunked_equals_one_shot(chunks):
    S, win = sum(chunks), 90
    w = W.make_batch(78, [S], [S], 8, 2, 128, "bf16", num_blocks=24)
    one = GpuState(w).step(w.steps[0], window=win)
    cw = W.chunked_steps(w, chunks)
    g = GpuState(cw)
    c = 0
    for st in cw.steps:
        o = g.step(st, window=win)
        n = st.num_tokens
        compare(o, one[c:c + n], "bf16", what=f"window chunk at {c}")
        c += n


@pytest.mark.timeout(600)
def test_window_c2_decode_batch():
    run_window(W.config2(), 1024, what="c2 W=1024")


@pytest.mark.timeout(600)
def test_window_c3_prefill_8k_every_tile():
    rows = tile_rows(0, 8192, 256, np.random.default_rng(5), n_random=24)
    run_window(W.config3(), 4096, rows=rows, what="c3 W=4096 rows of every tile")


@pytest.mark.timeout(600)
def test_window_c4_mixed_chunk_every_tile():
    w = W.config4()
    rows = np.concatenate([np.arange(30), tile_rows(30, 2048, 64, np.random.default_rng(6))])
    run_window(w, 4096, rows=rows, what="c4 W=4096 decodes + rows of every chunk tile")


@pytest.mark.timeout(600)
def test_window_c5_skewed_long_decode():
    run_window(W.config5(), 4096, what="c5 W=4096")
