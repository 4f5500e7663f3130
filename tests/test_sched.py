"""The C++ step planner (libpa, include/pa_sched.h) against the plain-Python oracle, step for step:
identical batches (every index array), identical pool and cache counters, identical preemptions.
Host code only: runs without a GPU."""
import numpy as np
import pytest

import attention_paged_kv_amd as pa
from attention_paged_kv_amd.sched import Planner
from oracle.sched_oracle import SchedOracle


def compare_step(cpp, orc, rng, stop_p):
    b = cpp.schedule()
    plan = orc.schedule()
    ids, qsl, seq_lens, tables, slots, toks, pos, samples = orc.step_arrays(plan)
    assert b.request_ids.tolist() == ids
    assert b.query_start_loc.tolist() == qsl
    assert b.seq_lens.tolist() == seq_lens
    assert b.block_tables.tolist() == tables
    assert b.slot_mapping.tolist() == slots
    assert b.token_ids.tolist() == toks
    assert b.positions.tolist() == pos
    assert b.samples.tolist() == samples
    assert b.max_q_len == (max(q1 - q0 for q0, q1 in zip(qsl, qsl[1:])) if len(qsl) > 1 else 0)
    assert cpp.preempted() == orc.preempted
    nxt = [int(x) for x in rng.integers(0, 40, len(plan))]
    stop = [int(x) for x in (rng.random(len(plan)) < stop_p)]
    cpp.commit(nxt, stop)
    orc.commit(nxt, stop)
    st, so = cpp.stats(), orc.stats()
    assert (st["free_blocks"], st["cached_blocks"], st["evictable_blocks"], st["running"], st["waiting"],
            st["hit_tokens"]) == (so["free"], so["cached"], so["evictable"], so["running"], so["waiting"],
                                  so["hit_tokens"])
    orc.check_invariants()
    return len(plan)


@pytest.mark.parametrize("seed,nb,mb,budget,max_seqs,prefix", [
    (0, 64, 16, 64, 0, True),
    (1, 12, 8, 48, 0, True),          # tight pool: eviction and preemption
    (2, 40, 12, 100, 6, True),
    (3, 40, 12, 100, 0, False),
    (4, 9, 9, 16, 3, True),
    (5, 256, 64, 512, 0, True),
])
def test_cpp_planner_matches_oracle(seed, nb, mb, budget, max_seqs, prefix):
    rng = np.random.default_rng(seed)
    cpp = Planner(nb, mb, budget, max_seqs=max_seqs, prefix_cache=prefix)
    orc = SchedOracle(nb, mb, budget, max_seqs=max_seqs, prefix_cache=prefix)
    prefixes = [[int(x) for x in rng.integers(0, 40, 48)] for _ in range(3)]
    rid = 0
    preempts = 0
    for step in range(400):
        if rng.random() < 0.35 and len(orc.by_id) < 24:
            pre = prefixes[int(rng.integers(0, 3))][: int(rng.integers(0, 48))]
            prompt = pre + [int(x) for x in rng.integers(0, 40, int(rng.integers(1, 40)))]
            max_new = int(rng.integers(1, 30))
            if len(prompt) + max_new <= mb * 16:
                cpp.add(rid, prompt, max_new)
                orc.add(rid, prompt, max_new)
                rid += 1
        if rng.random() < 0.02 and orc.by_id:
            victim = sorted(orc.by_id)[int(rng.integers(0, len(orc.by_id)))]
            cpp.abort(victim)
            orc.abort(victim)
        compare_step(cpp, orc, rng, 0.03)
        preempts += len(orc.preempted)
    if nb <= 12:
        assert preempts > 0
    if prefix:
        assert orc.hit_tokens > 0


def test_thirty_decodes_and_a_long_prompt_on_the_cpp_planner():
    """The P4 scenario, on the C++ planner: 15 steps, 30 decode tokens in each, totals <= budget."""
    p = Planner(4096, 2048, 2048)
    for i in range(30):
        p.add(i, [1000 + i] * 8, 10000)
    for _ in range(3):
        b = p.schedule()
        p.commit([7] * b.num_seqs)
    p.add(99, list(range(30000)), 5)
    steps = 0
    while True:
        b = p.schedule()
        steps += 1
        assert int((b.request_ids < 30).sum()) == 30 and b.num_tokens <= 2048
        k = int(np.where(b.request_ids == 99)[0][0])
        done = b.samples[k] == 1
        p.commit([7] * b.num_seqs)
        if done:
            break
    assert steps == 15


def test_planner_errors_leave_state_untouched():
    p = Planner(16, 4, 32)
    with pytest.raises(pa.PAError):
        p.add(1, [], 3)                                 # empty prompt
    with pytest.raises(pa.PAError):
        p.add(1, list(range(60)), 10)                   # longer than a block table (64 tokens)
    p.add(1, list(range(20)), 3)
    with pytest.raises(pa.PAError):
        p.add(1, [5], 1)                                # duplicate live id
    with pytest.raises(pa.PAError):
        p.commit([0])                                   # nothing planned
    b = p.schedule()
    assert b.num_seqs == 1
    with pytest.raises(pa.PAError):
        p.schedule()                                    # previous step not committed
    with pytest.raises(pa.PAError):
        p.abort(1)                                      # not between schedule and commit
    p.commit([3])
    with pytest.raises(pa.PAError):
        p.abort(77)                                     # unknown id
    with pytest.raises(pa.PAError):
        Planner(0, 4, 32)
    with pytest.raises(pa.PAError):
        Planner(16, 4, 0)


@pytest.mark.parametrize("seed,nb,budget,prefix", [(0, 40, 96, True), (1, 18, 64, True), (2, 40, 96, False)])
def test_planned_steps_on_the_paged_oracle_equal_attention_from_scratch(seed, nb, budget, prefix):
    """The planner's batches, run by the oracle over one shared paged cache (blocks reused across
    requests by the prefix cache, recycled after evictions, rewritten after preemption), give bit
    for bit what the oracle gives from scratch on a contiguous cache per request."""
    from tests.serving_helpers import OraclePagedExecutor, drive

    def check(out, ref, step, b):
        assert np.array_equal(out, ref), step
    c = drive(seed, nb, budget, prefix, OraclePagedExecutor(nb), check)
    assert c["steps"] > 20
    if prefix:
        assert c["hits"] > 0
    if nb < 20:
        assert c["preempts"] > 0
