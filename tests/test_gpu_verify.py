"""GPU parity of multi-token verification rows (P4 "一步的 token 预算": verifying a speculative draft
advances several tokens of a request in one step; P2 §4.3: a draft is checked in one pass of the
large model).  Requests with 2 <= q_len <= 8 run on the split-KV decode pass with (position, head)
columns, each column masked to its own causal (and window) range; they are compared with the CPU
oracle, mixed with plain decodes and with longer prompts that stay on the prefill tiles."""
import numpy as np
import pytest

import attention_paged_kv_amd as pa
from attention_paged_kv_amd import workloads as W
import oracle
from tests.gpu_helpers import GpuState, compare, host_array, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def check_mode():
    pa.set_check(True)
    yield
    pa.set_check(False)


def run(w, window=0, rows=None, what="", max_q_len=0):
    st = w.steps[0]
    g = GpuState(w)
    out_g = g.step(st, window=window, max_q_len=max_q_len)
    kc, vc = w.k_cache0.copy(), w.v_cache0.copy()
    out_r, _ = oracle.run_step(w, st, kc, vc, rows=rows, window=window)
    assert np.array_equal(host_array(g.kc, w.dtype), kc), f"{what}: K cache differs after append"
    compare(out_g, out_r, w.dtype, rows=rows, what=what)
    return out_g


CASES = [
    # seq_lens, q_lens, Hq, Hkv, d, window
    ([2], [2], 8, 8, 128, 0),
    ([17, 16, 33, 300], [2, 3, 8, 5], 8, 2, 128, 0),
    ([15, 31, 47, 63, 64, 65], [4, 4, 4, 4, 4, 4], 32, 32, 128, 0),      # keys of the last positions straddle blocks
    ([1000, 2048, 3001, 517], [8, 1, 7, 2], 32, 8, 128, 0),              # several splits, merge per position
    ([700, 129, 40], [6, 2, 8], 16, 1, 64, 0),                           # 16 heads per KV head: 128 columns
    ([1030, 260, 90], [1, 3, 90], 24, 3, 128, 0),                         # verify rows beside a prefill
    ([3000, 777, 64], [4, 8, 2], 32, 8, 128, 100),                        # windows start mid-block per column
    ([3000, 777, 64], [4, 8, 2], 32, 8, 128, 17),
    ([500, 500], [8, 8], 8, 2, 128, 1),
    ([9000], [8], 32, 8, 128, 0),
    # the first position's window reaches q_len - 1 keys further back than the last one's: with
    # W = 238 and q_len 8 a row's pass spans up to 260 keys, past one 256-key run
    ([3000, 1243, 250, 5000], [8, 8, 7, 8], 32, 8, 128, 238),
    # more than 64 rows: the run cursor walks several 64-row chunks of the batch
    ([100 + 37 * i for i in range(70)], [1 + i % 4 for i in range(70)], 8, 2, 128, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_verify_rows(case):
    seq, ql, Hq, Hkv, d, win = CASES[case]
    say(f"verify case {case}: seq {seq} q {ql} Hq {Hq} Hkv {Hkv} d {d} W {win}")
    nb = sum((s + 15) // 16 for s in seq) + 3
    w = W.make_batch(800 + case, seq, ql, Hq, Hkv, d, "bf16", num_blocks=nb)
    run(w, window=win, what=f"verify[{case}]")


def test_verify_rows_equal_one_token_steps():
    """A verify step over k new tokens equals k single-token steps (each appends then attends)."""
    w = W.make_batch(820, [600, 333], [6, 6], 16, 4, 128, "bf16", num_blocks=80)
    st = w.steps[0]
    one = GpuState(w).step(st)
    g = GpuState(w)
    for j in range(6):
        rows = np.array([j, 6 + j])
        sj = W.Step(q=st.q[rows], k_new=st.k_new[rows], v_new=st.v_new[rows], slot_mapping=st.slot_mapping[rows],
                    seq_lens=st.seq_lens - 5 + j, query_start_loc=np.array([0, 1, 2], np.int32),
                    block_tables=st.block_tables)
        o = g.step(sj)
        compare(o, one[rows], "bf16", what=f"token {j}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,k,hint", [("c2", 4, 0), ("c5", 8, 0), ("c2", 4, 4), ("c5", 4, 4)])
def test_verify_batches_at_decode_workload_sizes(cfg, k, hint):
    """Full-size verification steps, without and with the q_len bound the benchmark passes (the
    bound changes how many positions a row's columns are planned for)."""
    w = W.verify_variant(W.CONFIGS[cfg](), k)
    run(w, what=f"{cfg} verify {k} bound {hint}", max_q_len=hint)


def test_max_q_len_hint_skips_tiles_and_matches():
    """With the caller's bound on q_len (<= 8) the tile pass is not launched; results are those of
    the call without the bound.  A bound below some q_len is reported in check mode."""
    seq, ql, Hq, Hkv, d, win = CASES[3]
    w = W.make_batch(431, seq, ql, Hq, Hkv, d, "bf16", num_blocks=sum((s + 15) // 16 for s in seq) + 3)
    g0, g1 = GpuState(w), GpuState(w)
    pa.timing_reset()
    pa.timing_enable(True)
    try:
        ref = g0.step(w.steps[0])
        plain = pa.timing_read("prefill_tile")[1]
        out = g1.step(w.steps[0], max_q_len=max(ql))
        hinted = pa.timing_read("prefill_tile")[1] - plain
    finally:
        pa.timing_enable(False)
    assert plain == 1 and hinted == 0, (plain, hinted)
    assert np.array_equal(out, ref)
    pa.set_check(True)
    try:
        with pytest.raises(pa.PAError) as ei:
            GpuState(w).step(w.steps[0], max_q_len=max(ql) - 1)
        assert ei.value.code == 5 and "max_q_len" in str(ei.value)
    finally:
        pa.set_check(False)
