/*
 * pa_sched.h -- host-side step planner of libpa: the block pool, a token-budget scheduler and a
 * prefix cache, producing exactly the index arrays that pa_append_kv and pa_attention take
 * (slot_mapping, block_tables, seq_lens, query_start_loc).  Host code only: every pointer here is
 * host memory, nothing touches a device, and nothing is asynchronous.  Errors are pa_status codes
 * (pa.h) with the text in pa_last_error().
 *
 * Sources, cited by page and section:
 *   P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576), §2.2-2.3: fixed 16-token blocks
 *       from a free pool, addressed through a block table.
 *   P3  prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127),
 *       §4.3: prefix caching by exact token-sequence longest-prefix match, the matched K/V reused and
 *       only the suffix prefilled, positions continuing after the prefix, block-wise cache memory,
 *       LRU eviction by block rather than by request.
 *   P4  "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill), "一步的 token
 *       预算": per step a decoding request advances 1 token and a prefilling one min(remaining
 *       input, remaining budget), the step total stays within the budget, decodes go first;
 *       "把长输入切成块": a long prompt is cut into chunks that interleave with the decodes.
 *
 * Policy.  A request holds its token ids (prompt, then each sampled token), how many are computed
 * and its block list; it is decoding when its prompt is computed and exactly one token is pending.
 * pa_sched_schedule plans one step with budget = token_budget:
 *   1. decoding requests in admission order, 1 token each, while budget and the sequence cap
 *      allow.  A decode that needs a fresh block when the pool has none preempts the most recently
 *      admitted running request not yet in the step (possibly itself): its blocks are released,
 *      its computed count reset, and it goes to the front of the waiting queue to be recomputed;
 *   2. prefilling running requests in admission order, then (unless the step preempted) waiting
 *      requests in queue order: n = min(pending tokens, budget left), shrunk to what the pool can
 *      back; a waiting request that gets no token stops admission.
 * Admission first matches the prefix cache: at most (tokens - 1) / 16 full blocks, each looked up
 * by (parent cache entry, its 16 token ids), so at least one token is always computed and no
 * write ever lands in a shared block.  A block whose last holder releases it returns to the free
 * list, or, if it is cached, to the tail of the LRU list; allocation takes the free list first,
 * then evicts the LRU head.  Requests release their blocks last-first.  pa_sched_commit marks the
 * step's tokens computed, registers every block that became full under (parent entry, 16 token
 * ids) -- a parent entry is (block id, registration count), so a recycled block id never matches
 * old children -- appends the sampled token of each request whose step reached its last known
 * token, and finishes requests that reach max_new_tokens or that the caller stops.
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

typedef struct {
  int32_t num_blocks;          /* blocks in the pool (the cache's num_blocks)                    */
  int32_t max_blocks_per_seq;  /* block-table width; prompt + max_new_tokens <= 16 * this       */
  int32_t token_budget;        /* most tokens per step (>= 1)                                    */
  int32_t max_seqs;            /* most requests per step; 0 = no cap                             */
  int32_t prefix_cache;        /* 1: match and register full blocks; 0: never share blocks       */
} pa_sched_config;

/* One planned step, in caller-owned host arrays.  In: the capacities.  Out: the sizes and the
 * arrays, in step order (decodes first).  block_tables rows are padded with -1.  samples[i] = 1
 * when request i's scheduled tokens end at its last known token, so the step yields its next
 * token (passed back through pa_sched_commit).  The step's longest q_len (the largest difference of
 * consecutive query_start_loc entries) is the bound to pass as pa_attention_opts.max_q_len. */
typedef struct {
  int32_t cap_seqs;            /* in: >= max_seqs, or >= live requests when max_seqs == 0         */
  int32_t cap_tokens;          /* in: >= token_budget                                            */
  int32_t num_seqs;            /* out: B                                                          */
  int32_t num_tokens;          /* out: T                                                          */
  int64_t* request_ids;        /* [cap_seqs]                                                      */
  int32_t* query_start_loc;    /* [cap_seqs + 1]                                                  */
  int32_t* seq_lens;           /* [cap_seqs]: keys visible after the step's append               */
  int32_t* block_tables;       /* [cap_seqs][max_blocks_per_seq]                                  */
  int32_t* slot_mapping;       /* [cap_tokens]: block * 16 + offset of each scheduled token       */
  int32_t* token_ids;          /* [cap_tokens]                                                    */
  int32_t* positions;          /* [cap_tokens]                                                    */
  int32_t* samples;            /* [cap_seqs]                                                      */
} pa_sched_batch;

typedef struct {
  int32_t free_blocks;         /* never-cached or released uncached blocks                       */
  int32_t cached_blocks;       /* blocks registered in the prefix cache (held or evictable)      */
  int32_t evictable_blocks;    /* cached blocks nobody holds (the LRU list)                      */
  int32_t running;
  int32_t waiting;
  int32_t preempted_last_step;
  int64_t hit_tokens;          /* tokens taken from the prefix cache at admission, in total      */
} pa_sched_stats;

/* Creates a planner; *out = NULL and PA_ERR_INVALID_ARG for a bad configuration. */
int pa_sched_create(const pa_sched_config* cfg, pa_sched** out);
void pa_sched_destroy(pa_sched* s);

/* Queues a request.  prompt: host int32[prompt_len], copied.  Rejects a duplicate live id,
 * prompt_len < 1, max_new_tokens < 1, or prompt_len + max_new_tokens > 16 * max_blocks_per_seq. */
int pa_sched_add(pa_sched* s, int64_t request_id, const int32_t* prompt, int32_t prompt_len,
                 int32_t max_new_tokens);

/* Drops a live request and releases its blocks.  Not allowed between schedule and commit. */
int pa_sched_abort(pa_sched* s, int64_t request_id);

/* Plans one step into *batch (num_seqs may be 0).  The capacities are checked before any state
 * changes; a second schedule before commit is refused. */
int pa_sched_schedule(pa_sched* s, pa_sched_batch* batch);

/* Ends the planned step once its K/V are in the cache.  next_tokens: host int32[num_seqs], read
 * where samples[i] = 1; stop: NULL or host int32[num_seqs], nonzero finishes request i after its
 * sample. */
int pa_sched_commit(pa_sched* s, const int32_t* next_tokens, const int32_t* stop);

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* st);

/* Ids preempted by the last pa_sched_schedule: up to cap of them into ids, their count in *n. */
int pa_sched_preempted(const pa_sched* s, int64_t* ids, int32_t cap, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H_ */
