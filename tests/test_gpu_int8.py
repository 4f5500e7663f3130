"""GPU parity of the 8-bit KV cache (P2 §4.3, §5.4: INT8 codes with per-channel calibration) against
the CPU oracle: quantising append bit for bit over the whole cache, attention within the bf16
tolerances (decode rows, prompts, chunks over cached context, mixed steps), dequantised argmax
probes bit-exact."""
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


def run_i8(w, window=0, rows=None, what="", max_q_len=0):
    st = w.steps[0]
    g = GpuState(w)
    out_g = g.step(st, window=window, max_q_len=max_q_len)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    out_r, _ = oracle.run_step(w, st, kc, vc, rows=rows, window=window)
    assert np.array_equal(host_array(g.kc, "i8"), kc), f"{what}: K codes differ after append"
    assert np.array_equal(host_array(g.vc, "i8"), vc), f"{what}: V codes differ after append"
    compare(out_g, out_r, "bf16", rows=rows, what=what)
    return out_g


def i8_batch(seed, seq, Hq, Hkv, d, nb_extra=3):
    return W.make_batch(seed, seq, [1] * len(seq), Hq, Hkv, d, "bf16",
                        num_blocks=sum((s + 15) // 16 for s in seq) + nb_extra, cache="i8")


CASES = [
    # seq_lens (all decode rows), Hq, Hkv, d
    ([1], 1, 1, 128),
    ([15, 16, 17, 31, 32, 33], 8, 2, 128),
    ([47, 48, 49, 63, 64, 65], 4, 4, 64),
    ([255, 256, 257, 511, 512, 513], 32, 8, 128),
    ([1000, 2048, 3000], 32, 32, 128),
    ([700, 129, 5], 16, 1, 64),
    ([1030, 300], 24, 3, 128),
    ([4097, 9000], 64, 4, 128),
    ([2000, 33, 700], 64, 2, 128),          # 32 query heads per KV head
    # cache rows of 4 KiB or more (KV heads x d codes) are staged as whole rows of four heads:
    ([1, 15, 16, 17, 33, 700, 2500], 34, 34, 128),   # last head group holds two heads
    ([1, 17, 48, 321, 1500], 64, 64, 64),
    ([5, 260, 1100], 132, 66, 64),                   # d = 64, last group of two heads, 2 q-heads each
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_int8_decode_batches(case):
    seq, Hq, Hkv, d = CASES[case]
    say(f"int8 case {case}: seq {seq} Hq {Hq} Hkv {Hkv} d {d}")
    run_i8(i8_batch(600 + case, seq, Hq, Hkv, d), what=f"int8[{case}]")


@pytest.mark.parametrize("window", [1, 16, 17, 100, 1000])
def test_int8_decode_with_window(window):
    w = i8_batch(650 + window, [15, 16, 17, 600, 2000, 3001], 8, 2, 128)
    run_i8(w, window=window, what=f"int8 W={window}")


@pytest.mark.parametrize("window", [1, 17, 1000])
def test_int8_decode_with_window_whole_rows(window):
    w = i8_batch(680 + window, [15, 16, 17, 600, 2000, 3001], 64, 32, 128)
    run_i8(w, window=window, what=f"int8 whole rows W={window}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (64, 32)])
def test_int8_argmax_probe_bit_exact(Hq, Hkv):
    """Power-of-two scales make code * scale exact; with one dominant key per row the output is its
    dequantised V row, bit for bit, after the split merge too (per-wave and whole-row staging)."""
    d = 128
    lens = [67, 300, 1500, 16, 17]
    w = i8_batch(700, lens, Hq, Hkv, d)
    rng = np.random.default_rng(7)
    w.k_scale = (2.0 ** -rng.integers(4, 8, (Hkv, d))).astype(np.float32)
    w.v_scale = (2.0 ** -rng.integers(4, 8, (Hkv, d))).astype(np.float32)
    w.k_scale[:, 0] = 1.0
    st = w.steps[0]
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    kflat = kc.reshape(-1, Hkv, d)
    targets = []
    for b, s in enumerate(lens):
        slots = W.slots_for(st.block_tables, b, np.arange(s - 1))
        kflat[slots] = 0
        if s > 1:
            tgt = int(rng.integers(0, s - 1))
            kflat[slots[tgt], :, 0] = 127
            targets.append(slots[tgt])
        else:
            targets.append(None)
    knew = np.zeros((len(lens), Hkv, d), np.float32)
    qf = np.zeros((len(lens), Hq, d), np.float32)
    qf[:, :, 0] = 64.0
    st2 = W.Step(q=W.to_storage(qf, "bf16"), k_new=W.to_storage(knew, "bf16"), v_new=st.v_new,
                 slot_mapping=st.slot_mapping, seq_lens=st.seq_lens, query_start_loc=st.query_start_loc,
                 block_tables=st.block_tables)
    g = GpuState(w, kc, vc)
    out = g.step(st2)
    for b, tslot in enumerate(targets):
        if tslot is None:
            continue
        vt = vc.reshape(-1, Hkv, d)[tslot].astype(np.float32) * w.v_scale
        expect = np.repeat(W.to_storage(vt, "bf16"), Hq // Hkv, axis=0)
        assert np.array_equal(out[b], expect), b


@pytest.mark.parametrize("Hkv", [8, 32])
def test_int8_repeat_runs_bitwise_identical(Hkv):
    w = i8_batch(710, [3000, 47, 900], 32, Hkv, 128)
    a = GpuState(w).step(w.steps[0])
    b = GpuState(w).step(w.steps[0])
    assert np.array_equal(a, b)


PREFILL_CASES = [
    # seq_lens, q_lens, Hq, Hkv, d: one-shot prompts, chunks over cached context, mixes with decodes
    ([1, 2, 16, 17], [1, 2, 16, 17], 4, 2, 128),
    ([40, 20], [40, 1], 8, 2, 128),
    ([100, 64, 17, 129], [100, 64, 17, 129], 8, 8, 64),
    ([300, 1000], [37, 129], 16, 4, 128),
    ([500, 17, 3000, 64, 2], [1, 17, 200, 1, 2], 32, 8, 128),
    ([700, 257], [300, 256], 16, 1, 64),
    ([600, 2000, 33, 9], [4, 8, 2, 8], 32, 8, 128),      # verify-sized rows
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_int8_prefill_and_chunk_rows(case):
    seq, ql, Hq, Hkv, d = PREFILL_CASES[case]
    say(f"int8 prefill case {case}: seq {seq} q {ql} Hq {Hq} Hkv {Hkv} d {d}")
    w = W.make_batch(720 + case, seq, ql, Hq, Hkv, d, "bf16",
                     num_blocks=sum((s + 15) // 16 for s in seq) + 3, cache="i8")
    run_i8(w, what=f"int8 prefill[{case}]")


@pytest.mark.parametrize("window", [1, 17, 100])
def test_int8_chunk_rows_with_window(window):
    w = W.make_batch(740 + window, [300, 1000, 33, 900], [37, 129, 33, 1], 16, 4, 128, "bf16",
                     num_blocks=160, cache="i8")
    run_i8(w, window=window, what=f"int8 chunks W={window}")


@pytest.mark.timeout(600)
def test_int8_c3_prefill_8k_every_tile():
    """Every 256-row tile of the 8k prefill over an int8 cache (all KV heads): first and last rows,
    a row per wave, random rows."""
    rows = tile_rows(0, 8192, 256, np.random.default_rng(3), n_random=24)
    run_i8(W.config3(cache="i8"), rows=rows, what="c3 int8 rows of every tile")


@pytest.mark.timeout(600)
def test_int8_c4_mixed_chunk_every_tile():
    rows = np.concatenate([np.arange(30), tile_rows(30, 2048, 64, np.random.default_rng(4))])
    run_i8(W.config4(cache="i8"), rows=rows, what="c4 int8 decodes + rows of every chunk tile")


@pytest.mark.timeout(600)
def test_int8_c2_decode_batch():
    run_i8(W.config2(cache="i8"), what="c2 int8")


@pytest.mark.timeout(600)
def test_int8_c5_skewed_long_decode():
    run_i8(W.config5(cache="i8"), what="c5 int8")


@pytest.mark.timeout(600)
def test_int8_c5_window():
    run_i8(W.config5(cache="i8"), window=4096, what="c5 int8 W=4096")


I8_VERIFY_CASES = [
    # seq_lens, q_lens, Hq, Hkv, d, window: rows of a few tokens to verify on the int8 decode kernel,
    # each (position, head) column masked to its own causal and window range
    ([17, 16, 33, 300], [2, 3, 8, 5], 8, 2, 128, 0),
    ([1000, 2048, 3001, 517], [8, 1, 7, 2], 32, 8, 128, 0),     # several splits, merge per position
    ([700, 129, 40], [6, 2, 8], 16, 1, 64, 0),                  # 16 heads per KV head: 128 columns
    ([3000, 777, 64], [4, 8, 2], 32, 8, 128, 100),              # windows start mid-block per column
    ([3000, 1243, 250, 5000], [8, 8, 7, 8], 32, 8, 128, 238),   # first position reaches past a split
    ([500, 500], [8, 8], 8, 2, 128, 1),
    # rows whose last split holds only keys past the first positions (129 = 128 + 1, 257 = 256 + 1):
    # those columns see no key of that split, whose partial must then carry no weight
    ([129, 257, 513, 40], [2, 4, 8, 3], 32, 8, 128, 0),
    ([1030, 260, 90], [1, 3, 90], 24, 3, 128, 0),              # verify rows beside a prefill
    ([17, 300, 1000, 2049], [2, 8, 5, 1], 64, 32, 128, 0),     # whole-row staging, 2 heads per KV head
    ([3000, 777, 64], [4, 8, 2], 64, 32, 128, 100),
    # stream runs of more than 64 blocks (block ids taken 64 at a time), whole-row and per-wave
    ([9000, 8000], [8, 8], 256, 32, 128, 0),
    ([20000, 14000], [8, 5], 128, 8, 128, 0),
    # whole-row stream runs at d = 64, and with a last head group of two heads
    ([33, 500, 1200], [3, 8, 5], 128, 64, 64, 0),
    ([3000, 777, 40], [4, 8, 2], 128, 64, 64, 100),
    ([17, 900, 2100], [8, 2, 6], 68, 34, 128, 0),
]


@pytest.mark.parametrize("case", range(len(I8_VERIFY_CASES)))
def test_int8_verify_rows(case):
    seq, ql, Hq, Hkv, d, win = I8_VERIFY_CASES[case]
    say(f"int8 verify case {case}: seq {seq} q {ql} Hq {Hq} Hkv {Hkv} d {d} W {win}")
    w = W.make_batch(760 + case, seq, ql, Hq, Hkv, d, "bf16",
                     num_blocks=sum((s + 15) // 16 for s in seq) + 3, cache="i8")
    run_i8(w, window=win, what=f"int8 verify[{case}]")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("hint", [0, 4])
def test_int8_verify_at_decode_workload_size(hint):
    w = W.verify_variant(W.CONFIGS["c5"](cache="i8"), 4)
    say(f"int8 verify: c5 requests, 4 tokens each, q_len bound {hint}")
    run_i8(w, what=f"c5 int8 verify 4 bound {hint}", max_q_len=hint)
