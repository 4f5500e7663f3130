"""Plain-Python reference of the host-side step planner: block pool, token-budget scheduler and
prefix cache.  TEST INFRASTRUCTURE ONLY (imported by the tests); shares no code with the C++
planner in libpa.

Sources (cited by page and section):
  P3  prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127),
      §4.3: prefix caching -- exact token-sequence longest-prefix match, cached K/V reused and only
      the unmatched suffix prefilled, positions continue after the cached prefix, block-wise cache
      memory, LRU eviction by block rather than by request.
  P4  "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill), "一步的 token
      预算": each request records how many tokens are computed and how many exist; per step a
      decoding request gets 1 token, a prefilling one min(remaining input, remaining budget); the
      step total never exceeds the budget; decodes are scheduled first.
  P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576), §2.2-2.3: fixed 16-token blocks
      taken from a free pool, addressed through a block table.

Policy (the readings taken where the pages stop; the C++ planner follows the same):
  * A request holds its token ids (prompt, then every sampled token), the count already computed,
    and its block list.  It is decoding when all its prompt tokens are computed and exactly one
    token is pending (the last sampled one); otherwise it is prefilling (a recomputed request
    catches up by chunks).
  * schedule(): budget = token_budget.  (1) Decoding requests in admission order, 1 token each,
    while budget and the sequence cap allow.  A decode that needs a fresh block and finds none
    preempts the most recently admitted running request not yet in this step (possibly itself):
    its blocks are released, its computed count reset to 0, and it goes to the front of the
    waiting queue to be recomputed later.  (2) Prefilling running requests in admission order, then
    waiting requests in queue order: n = min(pending, budget left), shrunk to what the pool can
    back; a waiting request that can get no token stops admission (the queue is FIFO), and a step
    that preempted admits nothing.
  * Admission with the prefix cache: walk the prompt's full blocks, at most (len(tokens) - 1) // 16
    of them (at least one token is always computed, and never into a shared block), while the
    cache holds a block for (parent entry, 16 token ids); every hit is taken (refcount + 1) and its
    16 tokens count as computed.
  * Blocks: refcount per block; a block whose refcount drops to 0 goes back to the free list, or,
    if it is registered in the cache, to the end of the LRU list.  Allocation takes the front of the
    free list, else evicts the front (least recently released) of the LRU list and drops its cache
    entry.  A finished or preempted request releases its blocks last-first, so a sequence's tail
    blocks are evicted before its head.
  * commit(): the scheduled tokens become computed; every block that became full is registered
    under key (parent entry, its 16 token ids), where the parent entry is the cache entry of the
    request's previous block (or the root) as (block id, registration epoch) -- a block id alone
    could be reused for other content after an eviction.  If the key already names another block,
    the request keeps its block unregistered and chains on the existing entry.  A request whose
    scheduled tokens reached its last known token appends the sampled token; it finishes when it
    has max_new_tokens sampled tokens or the caller stops it, and releases its blocks.
"""
from __future__ import annotations

from collections import deque

BLOCK = 16
ROOT = (-1, 0)


class Req:
    def __init__(self, rid, prompt, max_new):
        self.rid = rid
        self.tokens = list(prompt)
        self.prompt_len = len(prompt)
        self.max_new = max_new
        self.generated = 0
        self.computed = 0
        self.blocks = []          # physical block ids, position order
        self.chain = []           # cache entry (block, epoch) standing for the prefix through block j
        self.admit_seq = -1

    @property
    def decoding(self):
        return self.computed >= self.prompt_len and len(self.tokens) - self.computed == 1


class SchedOracle:
    def __init__(self, num_blocks, max_blocks_per_seq, token_budget, max_seqs=0, prefix_cache=True):
        assert num_blocks >= 1 and max_blocks_per_seq >= 1 and token_budget >= 1
        self.nb, self.mb, self.budget, self.max_seqs = num_blocks, max_blocks_per_seq, token_budget, max_seqs
        self.prefix_cache = prefix_cache
        self.free = deque(range(num_blocks))
        self.lru = []                          # evictable cached blocks, least recently released first
        self.ref = [0] * num_blocks
        self.key_of = [None] * num_blocks       # cache key a block is registered under
        self.epoch = [0] * num_blocks           # registrations so far (part of child keys)
        self.cache = {}                         # key -> block
        self.waiting = deque()
        self.running = []                       # admission order
        self.by_id = {}
        self.pending = None
        self.admit_counter = 0
        self.preempted = []                     # request ids preempted by the last schedule()
        self.hit_tokens = 0

    # ---------------------------------------------------------------- pool
    def _alloc(self):
        if self.free:
            return self.free.popleft()
        if self.lru:
            b = self.lru.pop(0)
            del self.cache[self.key_of[b]]
            self.key_of[b] = None
            return b
        return None

    def _can_alloc(self, n):
        return len(self.free) + len(self.lru) >= n

    def _release_block(self, b):
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            if self.key_of[b] is not None:
                self.lru.append(b)
            else:
                self.free.append(b)

    def _release(self, r):
        for b in reversed(r.blocks):
            self._release_block(b)
        r.blocks = []
        r.chain = []

    def _take(self, b):
        if self.ref[b] == 0:
            self.lru.remove(b)
        self.ref[b] += 1

    # ---------------------------------------------------------------- requests
    def add(self, rid, prompt, max_new):
        if rid in self.by_id or len(prompt) < 1 or max_new < 1:
            raise ValueError("bad request")
        if len(prompt) + max_new > self.mb * BLOCK:
            raise ValueError("request longer than a block table")
        r = Req(rid, prompt, max_new)
        self.by_id[rid] = r
        self.waiting.append(r)

    def abort(self, rid):
        assert self.pending is None, "commit the previous step first"
        r = self.by_id.pop(rid)
        if r in self.running:
            self.running.remove(r)
        else:
            self.waiting.remove(r)
        self._release(r)

    def _blocks_needed(self, r, n):
        return (r.computed + n + BLOCK - 1) // BLOCK - len(r.blocks)

    def _grow(self, r, n):
        for _ in range(self._blocks_needed(r, n)):
            b = self._alloc()
            assert b is not None
            self.ref[b] += 1
            r.blocks.append(b)

    def _match(self, r):
        if not self.prefix_cache:
            return
        parent = ROOT
        limit = (len(r.tokens) - 1) // BLOCK
        for j in range(limit):
            key = (parent, tuple(r.tokens[j * BLOCK:(j + 1) * BLOCK]))
            b = self.cache.get(key)
            if b is None:
                break
            self._take(b)
            r.blocks.append(b)
            r.chain.append((b, self.epoch[b]))
            parent = (b, self.epoch[b])
        r.computed = len(r.blocks) * BLOCK
        self.hit_tokens += r.computed

    def _preempt(self, r):
        self.running.remove(r)
        self._release(r)
        r.computed = 0
        self.waiting.appendleft(r)
        self.preempted.append(r.rid)

    def schedule(self):
        """Plan one step; returns a list of (request id, first position, token count) in step order."""
        assert self.pending is None, "commit the previous step first"
        budget = self.budget
        plan = []
        in_step = set()
        self.preempted = []
        cap = self.max_seqs or (1 << 30)
        # (1) decodes
        for r in list(self.running):
            if r not in self.running or not r.decoding:
                continue
            if budget == 0 or len(plan) == cap:
                break
            while self._blocks_needed(r, 1) > 0 and not self._can_alloc(1):
                victims = [v for v in self.running if v.rid not in in_step]
                victim = max(victims, key=lambda v: v.admit_seq)
                self._preempt(victim)
                if victim is r:
                    break
            if r not in self.running:
                continue
            self._grow(r, 1)
            plan.append((r.rid, r.computed, 1))
            in_step.add(r.rid)
            budget -= 1
        # (2) prefills: running first, then the waiting queue
        for r in list(self.running):
            if r.decoding or r.rid in in_step:
                continue
            if budget == 0 or len(plan) == cap:
                break
            n = self._fit(r, min(len(r.tokens) - r.computed, budget))
            if n == 0:
                break
            self._grow(r, n)
            plan.append((r.rid, r.computed, n))
            in_step.add(r.rid)
            budget -= n
        while self.waiting and budget > 0 and len(plan) < cap and not self.preempted:
            r = self.waiting[0]
            self._match(r)
            n = self._fit(r, min(len(r.tokens) - r.computed, budget))
            if n == 0:
                self.hit_tokens -= r.computed
                self._release(r)
                r.computed = 0
                break
            self.waiting.popleft()
            r.admit_seq = self.admit_counter
            self.admit_counter += 1
            self.running.append(r)
            self._grow(r, n)
            plan.append((r.rid, r.computed, n))
            in_step.add(r.rid)
            budget -= n
        self.pending = plan
        return plan

    def _fit(self, r, n):
        """Largest m <= n whose new blocks the pool can back."""
        avail = len(self.free) + len(self.lru)
        while n > 0 and self._blocks_needed(r, n) > avail:
            n = min(n - 1, (len(r.blocks) + avail) * BLOCK - r.computed)
        return max(n, 0)

    def step_arrays(self, plan):
        """The attention call's arrays for a plan: (ids, qsl, seq_lens, tables, slots, token_ids, positions, samples)."""
        ids, qsl, seq_lens, tables, slots, toks, pos, samples = [], [0], [], [], [], [], [], []
        for rid, start, n in plan:
            r = self.by_id[rid]
            ids.append(rid)
            qsl.append(qsl[-1] + n)
            seq_lens.append(start + n)
            tables.append(r.blocks + [-1] * (self.mb - len(r.blocks)))
            for p in range(start, start + n):
                slots.append(r.blocks[p // BLOCK] * BLOCK + p % BLOCK)
                toks.append(r.tokens[p])
                pos.append(p)
            samples.append(1 if start + n == len(r.tokens) else 0)
        return ids, qsl, seq_lens, tables, slots, toks, pos, samples

    def commit(self, next_tokens, stop=None):
        """next_tokens[i] / stop[i] for the i-th planned request (used where it samples)."""
        plan = self.pending
        assert plan is not None
        self.pending = None
        for i, (rid, start, n) in enumerate(plan):
            r = self.by_id[rid]
            r.computed = start + n
            # register blocks that became full
            for j in range(len(r.chain), r.computed // BLOCK):
                parent = r.chain[j - 1] if j > 0 else ROOT
                key = (parent, tuple(r.tokens[j * BLOCK:(j + 1) * BLOCK]))
                b = r.blocks[j]
                if not self.prefix_cache:
                    r.chain.append((b, self.epoch[b]))
                    continue
                if key in self.cache:
                    e = self.cache[key]
                    r.chain.append((e, self.epoch[e]))
                else:
                    self.epoch[b] += 1
                    self.cache[key] = b
                    self.key_of[b] = key
                    r.chain.append((b, self.epoch[b]))
            if start + n == len(r.tokens):
                r.tokens.append(int(next_tokens[i]))
                r.generated += 1
                if r.generated >= r.max_new or (stop is not None and stop[i]):
                    self.running.remove(r)
                    del self.by_id[rid]
                    self._release(r)

    def stats(self):
        return dict(free=len(self.free), cached=len(self.cache), evictable=len(self.lru),
                    running=len(self.running), waiting=len(self.waiting), hit_tokens=self.hit_tokens)

    def check_invariants(self):
        live = [r for r in self.running]
        refs = [0] * self.nb
        for r in live:
            for b in r.blocks:
                refs[b] += 1
        assert refs == self.ref
        assert len(self.free) + len(self.lru) + sum(1 for x in self.ref if x > 0) == self.nb
        for b in self.lru:
            assert self.ref[b] == 0 and self.key_of[b] is not None
        for b in self.free:
            assert self.ref[b] == 0 and self.key_of[b] is None
        for k, b in self.cache.items():
            assert self.key_of[b] == k
