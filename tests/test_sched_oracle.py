"""Pins for the plain-Python step planner (block pool, token-budget scheduler, prefix cache).

Sources: P3 prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127),
§4.3 prefix caching; P4 "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill),
"一步的 token 预算" and "把长输入切成块".
"""
import numpy as np
import pytest

from oracle.sched_oracle import BLOCK, SchedOracle


def run_step(s, next_token=lambda rid, k: 7, stop=None):
    plan = s.schedule()
    arrays = s.step_arrays(plan)
    nxt = [next_token(rid, s.by_id[rid].generated) for rid, _, _ in plan]
    s.commit(nxt, stop)
    s.check_invariants()
    return plan, arrays


def finish_all(s, limit=100000):
    for _ in range(limit):
        if not s.running and not s.waiting:
            return
        run_step(s)
    raise AssertionError("did not finish")


def test_thirty_decodes_and_a_30k_prompt_take_15_steps():
    """P4: 30 users decoding plus a 30000-token prompt under a 2048-token budget: every step keeps
    one token per decoding user, the prompt is cut into chunks and done in 15 steps."""
    s = SchedOracle(num_blocks=4096, max_blocks_per_seq=2048, token_budget=2048)
    for i in range(30):
        s.add(i, [1000 + i] * 8, max_new=10000)
    while not all(r.decoding for r in s.running) or s.waiting:
        run_step(s)
    s.add(99, list(range(30000)), max_new=5)
    steps = 0
    while True:
        plan, arr = run_step(s)
        steps += 1
        decodes = [p for p in plan if p[0] < 30]
        assert len(decodes) == 30 and all(n == 1 for _, _, n in decodes)
        assert sum(n for _, _, n in plan) <= 2048
        big = [p for p in plan if p[0] == 99]
        assert len(big) == 1
        if arr[7][plan.index(big[0])]:          # the prompt's last token was computed: it samples
            break
    assert steps == 15


def test_shared_system_prompt_hit_rate_above_90_percent():
    """P3 §4.3: a 1500-token system prompt with a 100-token question; a second request with the
    same system prompt reuses the cached K/V of its whole blocks and prefills only the rest."""
    sys_prompt = list(range(5000, 6500))
    s = SchedOracle(num_blocks=1024, max_blocks_per_seq=128, token_budget=4096)
    s.add(1, sys_prompt + list(range(100)), max_new=1)
    finish_all(s)
    s.add(2, sys_prompt + list(range(200, 300)), max_new=1)
    plan, arr = run_step(s)
    rid, start, n = plan[0]
    assert rid == 2 and start == (1500 // BLOCK) * BLOCK == 1488 and n == 1600 - 1488
    hit = start / 1600
    assert hit > 0.9
    # positions continue after the cached prefix (P3 §4.3 second point)
    assert arr[6][0] == 1488 and arr[2][0] == 1600


@pytest.mark.parametrize("p", [0, 5, 15, 16, 17, 40, 63, 64, 99])
def test_match_is_exact_token_prefix(p):
    base = list(range(100, 200))
    s = SchedOracle(num_blocks=64, max_blocks_per_seq=16, token_budget=512)
    s.add(1, base, max_new=1)
    finish_all(s)
    other = list(base)
    other[p] = 9999
    s.add(2, other, max_new=1)
    plan, _ = run_step(s)
    assert plan[0][1] == min(p // BLOCK, (len(other) - 1) // BLOCK) * BLOCK


def test_identical_block_after_a_different_prefix_is_not_a_hit():
    s = SchedOracle(num_blocks=64, max_blocks_per_seq=16, token_budget=512)
    a = list(range(64))
    s.add(1, a, max_new=1)
    finish_all(s)
    b = [7] * 16 + a[16:]                 # blocks 1..3 equal a's, block 0 differs
    s.add(2, b, max_new=1)
    plan, _ = run_step(s)
    assert plan[0][1] == 0


def test_whole_prompt_cached_still_computes_its_last_block():
    s = SchedOracle(num_blocks=64, max_blocks_per_seq=16, token_budget=512)
    a = list(range(64))                    # exactly 4 blocks
    s.add(1, a, max_new=1)
    finish_all(s)
    s.add(2, a, max_new=1)
    plan, arr = run_step(s)
    assert plan[0][1] == 48 and plan[0][2] == 16
    # the written slots are in a block of its own, never in a shared one
    table = arr[3][0]
    assert all(s.ref[table[p // BLOCK]] == 1 for p in range(48, 64)) or s.by_id.get(2) is None


def test_lru_evicts_by_block_least_recently_released_first_and_never_a_held_block():
    s = SchedOracle(num_blocks=8, max_blocks_per_seq=8, token_budget=512)
    a = list(range(64))                    # 4 blocks
    s.add(1, a, max_new=1)
    finish_all(s)                          # blocks of 1 released tail first: LRU = [b3, b2, b1, b0]
    blocks_a = [b for b in range(8) if s.key_of[b] is not None]
    assert len(blocks_a) == 4 and len(s.free) == 4
    lru_before = list(s.lru)
    s.add(2, a[:32] + [555] * 8, max_new=5)   # shares blocks 0, 1 with a; holds them while running
    run_step(s)
    assert 2 in s.by_id and s.ref[lru_before[-1]] == 1 and s.ref[lru_before[-2]] == 1
    s.add(3, [321] * 70, max_new=5)        # needs 5 blocks: the free ones, then the LRU front
    run_step(s)
    r3 = s.by_id.get(3)
    taken = set(r3.blocks) if r3 else set()
    # the evicted cached block is a's tail block (released first), not one that request 2 holds
    assert lru_before[0] in taken
    assert not (taken & {lru_before[-1], lru_before[-2]})


def test_budget_decode_first_and_no_write_into_shared_blocks_random():
    rng = np.random.default_rng(0)
    s = SchedOracle(num_blocks=96, max_blocks_per_seq=32, token_budget=96, max_seqs=12)
    prefixes = [list(rng.integers(0, 50, 40)) for _ in range(4)]
    rid = 0
    for step in range(600):
        if rng.random() < 0.3 and len(s.by_id) < 30:
            pre = prefixes[rng.integers(0, 4)][: int(rng.integers(0, 40))]
            s.add(rid, pre + list(rng.integers(0, 50, int(rng.integers(1, 60)))), int(rng.integers(1, 40)))
            rid += 1
        n_dec = sum(1 for r in s.running if r.decoding)
        plan = s.schedule()
        arr = s.step_arrays(plan)
        assert sum(n for _, _, n in plan) <= 96 and len(plan) <= 12
        if not s.preempted:
            assert sum(1 for r, _, _ in plan if s.by_id[r].decoding) == min(n_dec, 12, 96)
        slots = arr[4]
        assert len(set(slots)) == len(slots)
        for r, start, n in plan:
            req = s.by_id[r]
            for p in range(start, start + n):
                assert s.ref[req.blocks[p // BLOCK]] == 1        # written blocks are private
        s.commit([int(rng.integers(0, 50)) for _ in plan], [int(rng.random() < 0.05) for _ in plan])
        s.check_invariants()
    assert s.hit_tokens > 0


def test_preempted_requests_are_recomputed_and_finish_with_their_tokens():
    rng = np.random.default_rng(1)
    s = SchedOracle(num_blocks=10, max_blocks_per_seq=10, token_budget=64)
    want = {}
    for i in range(6):
        s.add(i, list(rng.integers(0, 30, 20)), max_new=60)
        want[i] = None
    seen_preempt = False
    done = {}
    for _ in range(5000):
        if not s.running and not s.waiting:
            break
        plan = s.schedule()
        seen_preempt |= bool(s.preempted)
        toks = [1000 * rid + s.by_id[rid].generated for rid, _, _ in plan]
        for rid, _, _ in plan:
            done[rid] = s.by_id[rid]
        s.commit(toks)
        s.check_invariants()
    assert seen_preempt and not s.running and not s.waiting
    for rid, r in done.items():
        assert r.tokens[20:] == [1000 * rid + k for k in range(60)]
