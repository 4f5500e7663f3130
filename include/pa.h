/*
 * pa.h -- C ABI of libpa: causal self-attention over a 16-token-block paged KV cache on
 * AMD MI355X (gfx950).  One call family serves decode, one-shot prefill and chunked prefill
 * as a single varlen batch in which each request advances q_len tokens over its context.
 *
 * Sources, cited by page and section:
 *   P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576)
 *   P2  "大模型推理性能优化：Prefill与Decode瓶颈及KV缓存显存管理" (wmrh.cn/news/64708)
 *   P3  prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127)
 *   P4  "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill)
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must be device memory of the current HIP device;
 *     the library never frees or keeps them past the call (work already queued on `stream`
 *     aside).  Host-struct pointers (pa_cache_desc) are read during the call only.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Every call is
 *     asynchronous on that stream and makes no host synchronisation, except in check mode.
 *   - Return value: PA_OK (0) or a pa_status code.  On an error detected on the host nothing
 *     is launched and no output is touched; pa_last_error() then describes it.  No C++
 *     exception crosses this boundary.
 *   - Cache layout (both caches, same descriptor):  [num_blocks][16][num_kv_heads][head_dim],
 *     contiguous, element type `dtype`.  Token slot s lives at block s/16, offset s%16; one
 *     token's K (or V) for all KV heads is one contiguous row of num_kv_heads*head_dim
 *     elements.  Position-major rows are the layout P1 §3.2 reports as the faster one for
 *     decode reads; they also make the append a contiguous row copy.
 *   - Byte offsets are computed in 64 bits: a cache may exceed 2^31 bytes.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5
#define PA_BLOCK_SIZE 16

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* null or misaligned pointer, bad size or descriptor          */
  PA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, dtype, group size)     */
  PA_ERR_DEVICE = 3,        /* a HIP call or launch failed; pa_last_error() has its text    */
  PA_ERR_WORKSPACE = 4,     /* caller workspace smaller than pa_attention_workspace_size()  */
  PA_ERR_CHECK_FAILED = 5   /* check mode found an invalid index in device-side arguments   */
} pa_status;

/* PA_DTYPE_I8: 8-bit cache (P2 §4.3 and §5.4: an INT8 KV cache halves memory and bandwidth and
 * needs per-channel calibration).  Cache elements are int8 codes in [-127, 127] with one fp32
 * scale per (KV head, channel) for K and one for V; the value of a code is code * scale. */
typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1, PA_DTYPE_I8 = 2 } pa_dtype;

/* Describes both caches.  block_size must be 16 (P1 §2.3: 16 tokens per block, a 4096-token
 * prompt takes 256 blocks).  head_dim must be 64 or 128.  For F32 and BF16 caches the same dtype
 * is used for q, k, v, both caches and out; for I8 caches q, k, v and out are bf16.
 * Every device buffer passed to this library (tensors, caches, scales, workspace) must be 16-byte
 * aligned; a misaligned one is refused with PA_ERR_INVALID_ARG before anything is launched. */
typedef struct {
  int32_t num_blocks;     /* NB: physical blocks in the pool                                */
  int32_t block_size;     /* must be PA_BLOCK_SIZE                                          */
  int32_t num_kv_heads;   /* Hkv                                                            */
  int32_t head_dim;       /* d: 64 or 128                                                   */
  int32_t dtype;          /* pa_dtype of the cache elements                                 */
  const float* k_scale;   /* I8 only: device fp32 [Hkv][d], finite and > 0 (caller's          */
  const float* v_scale;   /*   calibration); must be NULL for the other dtypes              */
} pa_cache_desc;

/* ABI version compiled into the library; a binding must refuse to run if it differs from
 * PA_ABI_VERSION (P1 §5.1 reports mismatched attention builds that silently return zeros). */
int pa_abi_version(void);

/* Text of the last error raised on the calling thread; valid until the next pa_* call on
 * that thread.  Empty string if none. */
const char* pa_last_error(void);

/* Frees the library-owned workspaces of every device (those used when pa_attention gets a
 * NULL workspace) and the side streams of mixed batches.  Synchronises the devices that own them. */
void pa_release(void);

/* Check mode: when on (or when the environment variable PA_CHECK=1 is set at the first call),
 * pa_attention and pa_append_kv first run a validator kernel over the index arguments,
 * synchronise `stream`, and return PA_ERR_CHECK_FAILED with the first offending index in
 * pa_last_error() instead of launching with invalid indices.  Off by default. */
void pa_set_check(int on);

/*
 * KV append -- P3 §2.3 (only K and V are cached, never Q), P1 §2.2 (each token's K/V are
 * written at their page index), P3 §3.1 (a decode step appends its K/V before attending),
 * P4 "把长输入切成块" (a prefill chunk writes its own K/V after reading the earlier ones).
 *
 *   k, v          device, [num_tokens][Hkv][d] contiguous, cache->dtype (bf16 for I8 caches).  Must
 *                 not alias the caches.
 *   slot_mapping  device int32 [num_tokens]: destination slot of each token (block*16 + offset);
 *                 a negative slot skips that token (padding).  Slots must lie in [0, NB*16) and be
 *                 distinct; otherwise the result is undefined (check mode reports it).
 *   k_cache,
 *   v_cache       device, layout above; row `slot` of each is overwritten bit for bit, all other
 *                 bytes are left untouched.  I8 caches: element c of head g is written as the code of
 *                 x = k[i][g][c] under s = k_scale[g][c] (v likewise): x / s rounded to fp32 (IEEE
 *                 division), then to the nearest integer with ties to even, clamped to [-127, 127];
 *                 NaN gives 0.
 * num_tokens == 0 is a no-op returning PA_OK.
 */
int pa_append_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                 void* k_cache, void* v_cache, const pa_cache_desc* cache, void* stream);

/* Workspace bytes pa_attention needs for a batch of these sizes (an upper bound computed from
 * the sizes alone; host-only, no device work).  Returns 0 for invalid sizes. */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_q_tokens, int32_t max_blocks_per_seq,
                                   int32_t num_q_heads, const pa_cache_desc* cache);

/*
 * Causal attention of a varlen batch over the paged cache -- P3 §2.1 (causal mask: position i
 * sees keys 0..i; softmax over scaled scores; weights multiply V), P3 §3.1 and §5.1 (decode:
 * q attends over all S+t cached keys after the append), P4 "一步的 token 预算" (each request
 * advances q_len tokens per step: decode, prefill and chunked prefill are one operation),
 * P3 §2.3 and §6.3 (grouped-query attention: Hq/Hkv query heads share one KV head).
 *
 * For request b: its query tokens are rows query_start_loc[b] .. query_start_loc[b+1]-1 of q;
 * q_len = their count, ctx = seq_lens[b] - q_len; query row r (0-based within the request) sits
 * at absolute position ctx + r and attends to keys 0 .. ctx + r, read through block_tables[b].
 * Query head h uses KV head h / (Hq/Hkv).
 *   out[t][h][:] = sum_j softmax_j(scale * <q[t][h], K[j][g]>) * V[j][g]
 * where for I8 caches K[j][g][c] = code * k_scale[g][c] and V likewise (q and out are bf16).  The
 * product q[c] * k_scale[g][c] is rounded once before it meets the codes: to fp16 after scaling
 * each query head by a power of two on the split-KV pass (rows of q_len <= 8), to bf16 on the
 * prefill tiles (longer rows); both are rounding choices inside the bf16 tolerance.
 *
 *   q                device [num_q_tokens][num_q_heads][d], cache->dtype.
 *   k_cache, v_cache device, layout above (already holding this step's appended K/V).
 *   block_tables     device int32 [num_seqs][max_blocks_per_seq]; entries past ceil(seq_len/16)
 *                    are never read (any value).
 *   seq_lens         device int32 [num_seqs]: keys visible to the request's last query token,
 *                    this step's tokens included; 1 <= q_len <= seq_len <= max_blocks_per_seq*16.
 *   query_start_loc  device int32 [num_seqs+1]: 0, then nondecreasing, ending at num_q_tokens;
 *                    every request has q_len >= 1 (so num_q_tokens >= num_seqs).
 *   scale            softmax scale, finite and > 0 (1/sqrt(d) for standard attention).
 *   out              device [num_q_tokens][num_q_heads][d], cache->dtype; must not alias inputs.
 *                    Accumulation is fp32 for both dtypes; bf16 output is rounded to nearest even.
 *   workspace        device scratch of at least pa_attention_workspace_size() bytes, owned by
 *                    the caller and not used concurrently by another call; NULL = use a
 *                    library-owned buffer of this (device, stream) pair.  Calls on one stream
 *                    share it safely (stream order); growing it synchronises that stream, then
 *                    frees and reallocates it (hipMalloc).  Such buffers live until pa_release().
 * Device-side index errors (bad q_len/seq_len, block id outside [0, NB)) are undefined unless
 * check mode is on.  num_q_heads must be a multiple of Hkv; for bf16, Hq/Hkv <= 128.
 * A batch with both decode rows (q_len <= 8 for bf16 activations, q_len 1 for fp32) and longer
 * rows (P4 "一步的 token 预算": all decodes plus a prefill chunk in one step) runs its decode pass on
 * a library-owned side stream of the device, forked from `stream` and joined back to it with
 * events: every kernel of the call still completes before later work on `stream` starts.
 */
int pa_attention(const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                 const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                 const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                 const int32_t* seq_lens, const int32_t* query_start_loc, float scale, void* out,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Options of pa_attention_ex.  A zeroed struct (or a NULL pointer) gives pa_attention's result. */
typedef struct {
  /* Sliding window (P2 §5.2 and P3 §6.3: keep only the most recent W tokens' K/V).  0: none.
   * W > 0: the query row at position p attends to keys max(0, p - W + 1) .. p only, itself
   * included, so W = 1 returns each row's own V.  Block-table entries of blocks that lie wholly
   * before the first query row's window, max(0, ctx - W + 1) with ctx = seq_len - q_len, are never
   * read (any value: a cache may drop such blocks), nor are the cache slots they would name.
   * Negative values are rejected with PA_ERR_INVALID_ARG. */
  int32_t sliding_window;
  /* Largest q_len of any request in the batch, when the caller knows it (a scheduler does).  0:
   * not given, the library assumes num_q_tokens - num_seqs + 1.  With a bound <= 8 (decode and
   * verification steps) the prefill-tile pass is not launched at all.  A request whose q_len
   * exceeds the bound gets an undefined output row; check mode reports it (PA_ERR_CHECK_FAILED).
   * Negative values are rejected with PA_ERR_INVALID_ARG. */
  int32_t max_q_len;
} pa_attention_opts;

/*
 * pa_attention with options; same arguments, layouts, ownership and errors, plus `opts` (host,
 * read during the call only; NULL = no options).  pa_attention_workspace_size() for the same
 * sizes is enough for every option value (a window only shrinks what is needed).
 */
int pa_attention_ex(const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                    const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                    const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* query_start_loc, float scale, void* out,
                    void* workspace, size_t workspace_bytes, const pa_attention_opts* opts, void* stream);

/* Bytes of the per-device scratch array behind pa_attention_noalloc (64 MiB). */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pa_attention_ex without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * layouts, ownership, results and errors as pa_attention_ex; the split partials and the tile list
 * live in a fixed array of PA_NOALLOC_SCRATCH_BYTES in each device's memory, held by the library
 * until the process ends.  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine; check mode also reports through that array).
 *   - A batch whose workspace would exceed PA_NOALLOC_SCRATCH_BYTES - 256 bytes is refused with
 *     PA_ERR_WORKSPACE before anything is launched (pa_attention_workspace_size() bounds the need).
 *   - Every call on a device shares that device's array, and each call overwrites what it uses
 *     (nothing in it needs to start at zero): calls that may overlap on one device -- on two
 *     streams, or from two threads -- race and must be serialised by the caller.
 */
int pa_attention_noalloc(const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                         const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                         const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* query_start_loc, float scale, void* out,
                         const pa_attention_opts* opts, void* stream);

/*
 * Measurement support (not part of the computation).  When timing is on, every kernel the
 * library launches is bracketed by a pair of hipEvents recorded on the same stream.
 * pa_timing_read() waits for the recorded events and returns, for the kernel family `name`
 * ("append", "decode_split", "decode_merge", "prefill_tile", "check"), the summed
 * duration in milliseconds and the number of launches since the last reset.
 */
int pa_timing_enable(int on);
int pa_timing_read(const char* name, double* total_ms, int64_t* launches);
void pa_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
