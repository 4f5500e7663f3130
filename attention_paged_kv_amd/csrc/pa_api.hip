// pa_api.hip -- the C ABI declared in include/pa.h: argument validation on the host, workspace
// layout, launch sequencing on the caller's stream, check mode, kernel timing and error text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <map>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_error.h"
#include "pa_internal.h"

namespace {
thread_local std::string g_err;
}  // namespace

namespace pa {
int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
void clear_error() { g_err.clear(); }
}  // namespace pa

namespace {

template <class... A>
int fail(int code, const char* fmt, A... args) {
  return pa::set_error(code, fmt, args...);
}

int device_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

std::atomic<int> g_check{-1};
bool check_on() {
  int v = g_check.load();
  if (v < 0) {
    const char* e = std::getenv("PA_CHECK");
    v = (e && e[0] == '1') ? 1 : 0;
    int expected = -1;
    g_check.compare_exchange_strong(expected, v);
    v = g_check.load();
  }
  return v == 1;
}

// Keys per decode split: PA_SPLIT_TOKENS if set (a multiple of 16 up to 1024), else 256 (320 over
// an 8-bit cache, ten of its 32-key units), or 384 when a row may span more than 8192 keys
// (measured: c5's rows of up to 32768 keys 175 against 179 us; c2's rows of up to 4096 keys 207
// against 211, and over an 8-bit cache 111 against 114 at 256).  `bound`: sizing a workspace that
// must serve every window and cache, so the smallest split (the most partials) is assumed.
int split_tokens(int64_t span, bool bound, bool i8) {
  static const int over = [] {
    const char* e = std::getenv("PA_SPLIT_TOKENS");
    const int s = e ? std::atoi(e) : 0;
    return (s >= 16 && s <= 1024 && s % 16 == 0) ? s : 0;   // <= 64 blocks per split
  }();
  if (over) return over;
  if (bound) return pa::kDefaultSplitTokens;
  if (span > 8192) return pa::kLongSplitTokens;
  return i8 ? pa::kI8SplitTokens : pa::kDefaultSplitTokens;
}

// ---- per-device state: the check-mode result slot and the compute-unit count ----
struct DevState {
  int* check = nullptr;
  int cus = 0;            // compute units
};
std::mutex g_dev_mu;
std::unordered_map<int, DevState> g_dev;

// ---- library-owned workspaces (calls given a NULL workspace): one per (device, stream) ----
// Calls on one stream run in stream order, so a buffer used by one stream only is never in use
// by two kernels at once.  g_ws_mu is held from the lookup until every kernel of the call is
// queued: a buffer is only grown (old one freed after its stream has drained) while no other
// call on that stream can be between its lookup and its launches.
struct StreamWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, uintptr_t>, StreamWs> g_ws;

// ---- kernel timing ----
struct TimedLaunch {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_t_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_pending;
std::vector<hipEvent_t> g_event_pool;
std::unordered_map<std::string, std::pair<double, int64_t>> g_t_acc;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  std::unique_lock<std::mutex> lk(g_t_mu);
  if (!g_timing) {
    lk.unlock();
    return launch();
  }
  hipEvent_t a = take_event(), b = take_event();
  hipError_t e = (a && b) ? hipEventRecord(a, s) : hipErrorOutOfMemory;
  if (e == hipSuccess) {
    e = launch();
    const hipError_t eb = hipEventRecord(b, s);
    if (e == hipSuccess) e = eb;
  }
  if (e == hipSuccess) {
    g_pending.push_back({name, a, b});
  } else {                                  // keep the events for later launches
    if (a) g_event_pool.push_back(a);
    if (b) g_event_pool.push_back(b);
  }
  return e;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Where each piece of an attention call lives in the workspace, and what runs.
struct Plan {
  bool bf16 = false;      // bf16 activations (bf16 or int8 cache)
  bool i8 = false;        // int8 cache
  int head_dim = 0, group = 0, heads_per_wg = 0;
  bool run_decode = false, run_tiles = false;
  int rows = 0, per_token = 0, qmax = 1, split = 0, max_splits = 0;
  bool stream = false;    // bf16 or int8 cache, rows of several positions: balanced runs, not splits
  int span_blocks = 0;    // most 16-key blocks one row's decode pass covers
  int pos_per_tile = 0, num_slots = 0;
  size_t off_o = 0, off_ml = 0, total = 0;
};

// The kernels move data in 16-byte vectors.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int validate_desc(const pa_cache_desc* c) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->block_size != PA_BLOCK_SIZE) return fail(PA_ERR_INVALID_ARG, "block_size must be 16 (got %d)", c->block_size);
  if (c->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1 (got %d)", c->num_blocks);
  if (c->num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", c->num_kv_heads);
  if (c->dtype != PA_DTYPE_F32 && c->dtype != PA_DTYPE_BF16 && c->dtype != PA_DTYPE_I8)
    return fail(PA_ERR_UNSUPPORTED, "unsupported dtype %d", c->dtype);
  if (c->dtype == PA_DTYPE_I8 && (!c->k_scale || !c->v_scale))
    return fail(PA_ERR_INVALID_ARG, "an int8 cache needs k_scale and v_scale");
  if (c->dtype != PA_DTYPE_I8 && (c->k_scale || c->v_scale))
    return fail(PA_ERR_INVALID_ARG, "k_scale / v_scale are for int8 caches only");
  if (misaligned(c->k_scale) || misaligned(c->v_scale))
    return fail(PA_ERR_INVALID_ARG, "k_scale / v_scale must be 16-byte aligned");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  return PA_OK;
}

// window: keys a row sees (pa::kNoWindow for all); it only bounds how many splits a row needs.
// max_q_len: the caller's bound on every q_len (0: none given).  bound: the plan only sizes a
// workspace for every option value.
int make_plan(int32_t B, int32_t T, int32_t MB, int32_t Hq, const pa_cache_desc* c, int window, int max_q_len,
              Plan& p, bool bound = false) {
  int rc = validate_desc(c);
  if (rc) return rc;
  if (B < 1) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", B);
  if (T < B) return fail(PA_ERR_INVALID_ARG, "num_q_tokens (%d) < num_seqs (%d): every request needs q_len >= 1", T, B);
  if (MB < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1 (got %d)", MB);
  if ((int64_t)MB * PA_BLOCK_SIZE > (1 << 30)) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  if (Hq < 1 || Hq % c->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", Hq, c->num_kv_heads);
  p.i8 = c->dtype == PA_DTYPE_I8;
  p.bf16 = c->dtype == PA_DTYPE_BF16 || p.i8;
  p.head_dim = c->head_dim;
  p.group = Hq / c->num_kv_heads;
  // A request row of bf16 activations (bf16 or int8 cache) carries up to qmax positions:
  // min(kVerifyMax, the longest q_len the sizes allow); fp32 rows carry one.  The matrix-core
  // decode kernels hold up to 16 (position, query head) columns of a KV head per wave (the MFMA
  // column count); the fp32 vector-ALU decode holds a divisor of the group size up to 8.
  const int longest = (max_q_len > 0 && max_q_len < T - B + 1) ? max_q_len : T - B + 1;
  p.qmax = p.bf16 ? (longest < pa::kVerifyMax ? longest : pa::kVerifyMax) : 1;
  if (p.bf16) p.heads_per_wg = p.qmax * p.group < 16 ? p.qmax * p.group : 16;
  else p.heads_per_wg = (p.group % 8 == 0) ? 8 : (p.group % 4 == 0) ? 4 : (p.group % 2 == 0) ? 2 : 1;
  if (p.bf16 && p.group > pa::kMaxTileGroup)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head (%d) above %d", p.group, pa::kMaxTileGroup);
  // A row's pass covers keys from the block holding the oldest key its first position sees (that
  // position's window reaches qmax - 1 keys further back than the last one's) to its last key:
  // at most min(MB * 16, window + qmax - 1 + 15) keys, and min(MB, ceil((window + qmax - 1) / 16) + 1)
  // blocks.
  const int64_t reach = (int64_t)window + p.qmax - 1;
  const int64_t span = std::min<int64_t>((int64_t)MB * PA_BLOCK_SIZE, reach + PA_BLOCK_SIZE - 1);
  p.span_blocks = (int)std::min<int64_t>(MB, (reach + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE + 1);
  // Rows of several positions (verification) make uneven work per split (more columns on some
  // rows, longer merges); they are dealt out in balanced runs.  Plain decode rows measure best on
  // fixed splits, which the hardware schedules dynamically.
  p.split = split_tokens(span, bound, c->dtype == PA_DTYPE_I8);
  p.stream = (c->dtype == PA_DTYPE_BF16 || c->dtype == PA_DTYPE_I8) && p.qmax > 1;
  if (p.stream) {
    // a row meets at most ceil(blocks / run) + 1 runs, and runs hold at least `split` keys
    p.max_splits = (int)(((int64_t)p.span_blocks * PA_BLOCK_SIZE + p.split - 1) / p.split) + 1;
    if ((int64_t)B * p.span_blocks > 0x7FFFFFFF) return fail(PA_ERR_UNSUPPORTED, "batch too large for one launch");
  } else {
    p.max_splits = (int)((span + p.split - 1) / p.split);
  }
  if (p.bf16) {
    p.per_token = 0;
    p.rows = B;
    p.run_decode = !(B == 1 && T > p.qmax);      // some request may have q_len <= qmax
    p.run_tiles = longest > p.qmax;              // some request may have q_len > qmax
    p.pos_per_tile = pa::kTileRows / p.group;
    p.num_slots = (T + p.pos_per_tile - 1) / p.pos_per_tile + B;
  } else {
    p.per_token = 1;
    p.rows = T;
    p.run_decode = true;
    p.run_tiles = false;
  }
  size_t off = 0;
  if (p.run_decode && p.max_splits > 1) {
    const size_t units = (size_t)p.rows * p.qmax * p.max_splits * Hq;
    p.off_o = off;
    off = align256(off + units * p.head_dim * sizeof(float));
    p.off_ml = off;
    off = align256(off + units * 2 * sizeof(float));
  }
  p.total = off;
  const int64_t nzh = ((int64_t)p.qmax * p.group + p.heads_per_wg - 1) / p.heads_per_wg;
  // KV heads per decode workgroup: 4 (int8), 2 or 4 (bf16: the smaller bounds the grid), 1 (fp32)
  const int64_t heads = p.i8 ? (c->num_kv_heads + 3) / 4 : p.bf16 ? (c->num_kv_heads + 1) / 2 : c->num_kv_heads;
  const int64_t dec_grid = heads * nzh * p.max_splits * p.rows;
  if (p.run_decode && !p.stream && dec_grid > 0x7FFFFFFF) return fail(PA_ERR_UNSUPPORTED, "batch too large for one launch");
  return PA_OK;
}

int get_device(int& dev) {
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  return PA_OK;
}

// Compute units of the current device (looked up once per device).
int chip_cus(int& cus) {
  int dev = 0;
  int rc = get_device(dev);
  if (rc) return rc;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    cus = g_dev[dev].cus;
  }
  if (cus == 0) {
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus < 1) return device_fail(e != hipSuccess ? e : hipErrorInvalidValue, "compute unit count");
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev[dev].cus = cus;
  }
  return PA_OK;
}

// Stream-mode workgroups per head group (bf16: two KV heads, their column groups carried inside
// the workgroup; int8: four KV heads and one column group): both decode kernels keep two workgroups
// resident per compute unit, so two per CU over all head groups make one full wave of the chip;
// never more than the rows' blocks fill with runs of `split` keys.  PA_DECODE_WGS overrides the
// chip-wide count.
int stream_wgs(const Plan& p, int num_kv_heads, int& out) {
  int cus = 0;
  int rc = chip_cus(cus);
  if (rc) return rc;
  static const int over = [] {
    const char* e = std::getenv("PA_DECODE_WGS");
    return e ? std::atoi(e) : 0;
  }();
  const int64_t nzh = ((int64_t)p.qmax * p.group + p.heads_per_wg - 1) / p.heads_per_wg;
  const int64_t nq = p.i8 ? (int64_t)((num_kv_heads + 3) / 4) * nzh : (num_kv_heads + 1) / 2;
  const int64_t chip = over > 0 ? over : 2 * (int64_t)cus;
  const int64_t fill = ((int64_t)p.rows * p.span_blocks * PA_BLOCK_SIZE + p.split - 1) / p.split;
  out = (int)std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(1, chip / nq), fill));
  return PA_OK;
}

int ensure_check_slot(int dev, int*& slot) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevState& st = g_dev[dev];
  if (!st.check) {
    hipError_t e = hipMalloc(&st.check, 4 * sizeof(int));
    if (e != hipSuccess) return device_fail(e, "hipMalloc(check)");
  }
  slot = st.check;
  return PA_OK;
}

// Validator kernel over the index arguments; `slot` (4 ints of device memory) receives its
// result, or the device's own slot is used when it is null.
int run_check(const pa::CheckArgs& base, hipStream_t s, int* slot = nullptr) {
  int rc;
  if (!slot) {
    int dev = 0;
    rc = get_device(dev);
    if (rc) return rc;
    rc = ensure_check_slot(dev, slot);
    if (rc) return rc;
  }
  pa::CheckArgs a = base;
  a.result = slot;
  hipError_t e = hipMemsetAsync(slot, 0, 4 * sizeof(int), s);
  if (e != hipSuccess) return device_fail(e, "hipMemsetAsync(check)");
  e = timed("check", s, [&] { return pa::launch_check(a, s); });
  if (e != hipSuccess) return device_fail(e, "check kernel");
  int host[4] = {0, 0, 0, 0};
  e = hipMemcpyAsync(host, slot, sizeof host, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_fail(e, "check readback");
  if (!host[0]) return PA_OK;
  static const char* what[] = {"", "slot outside the pool", "slot written twice", "query_start_loc[0] != 0",
                               "query_start_loc[num_seqs] != num_q_tokens", "q_len < 1", "seq_len < q_len",
                               "seq_len > max_blocks_per_seq*16", "block id outside [0, num_blocks)",
                               "q_len > max_q_len"};
  const int code = host[1] >= 1 && host[1] <= 9 ? host[1] : 0;
  return fail(PA_ERR_CHECK_FAILED, "check mode: %s (index %d, value %d)", what[code], host[2], host[3]);
}

// The arguments of one attention call.
struct Call {
  const void* q;
  int32_t T, Hq;
  const void* k_cache;
  const void* v_cache;
  const pa_cache_desc* cache;
  const int32_t* block_tables;
  int32_t B, MB;
  const int32_t* seq_lens;
  const int32_t* qsl;
  float scale;
  void* out;
  int window, max_q_len;
};

// Host checks shared by every attention entry point, and the plan of the call.
int prepare(const Call& c, const pa_attention_opts* opts, Call& full, Plan& p) {
  full = c;
  full.window = pa::kNoWindow;
  full.max_q_len = 0;
  if (opts) {
    if (opts->sliding_window < 0)
      return fail(PA_ERR_INVALID_ARG, "sliding_window must be >= 0 (got %d)", opts->sliding_window);
    if (opts->sliding_window > 0 && opts->sliding_window < pa::kNoWindow) full.window = opts->sliding_window;
    if (opts->max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "max_q_len must be >= 0 (got %d)", opts->max_q_len);
    full.max_q_len = opts->max_q_len;
  }
  int rc = make_plan(c.B, c.T, c.MB, c.Hq, c.cache, full.window, full.max_q_len, p);
  if (rc) return rc;
  if (!c.q || !c.k_cache || !c.v_cache || !c.block_tables || !c.seq_lens || !c.qsl || !c.out)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (c.out == c.q || c.out == c.k_cache || c.out == c.v_cache) return fail(PA_ERR_INVALID_ARG, "out must not alias inputs");
  if (misaligned(c.q) || misaligned(c.k_cache) || misaligned(c.v_cache) || misaligned(c.out))
    return fail(PA_ERR_INVALID_ARG, "q, the caches, out and the workspace must be 16-byte aligned");
  // the kernels track the running max of raw scores and apply the scale afterwards, which needs
  // scale > 0
  if (!std::isfinite(c.scale) || !(c.scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)c.scale);
  return PA_OK;
}

// ---- the side stream of a mixed step (decode rows beside prefill tiles), one per device ----
// A batch with both decode rows and prefill tiles queues its tile pass on the caller's stream and
// its decode pass (splits and merge) on this stream, forked from and joined back to the caller's
// stream by events, so that decode workgroups take compute units as soon as tile workgroups leave
// them instead of waiting for the whole tile pass (or holding it back).  The stream has the default
// priority.  g_side_mu serialises the fork-join sequences of concurrent calls (the events are reused).
std::mutex g_side_mu;
struct Side { hipStream_t s = nullptr; hipEvent_t fork = nullptr, join = nullptr; };
std::unordered_map<int, Side> g_side;
int side_stream(hipStream_t& s, hipEvent_t& fork, hipEvent_t& join) {
  int dev = 0;
  int rc = get_device(dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(g_side_mu);
  Side& sd = g_side[dev];
  if (!sd.s) {
    hipError_t e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming);
    if (e != hipSuccess) return device_fail(e, "side stream");
  }
  s = sd.s; fork = sd.fork; join = sd.join;
  return PA_OK;
}

// Queues the call's kernels on `s` (a mixed batch forks its decode pass to the side stream), with
// `ws` holding at least p.total bytes (null when p.total is 0).  Allocates nothing when
// `check_slot` is given (check mode then reports through it, and nothing is forked).
int launch_call(const Call& c, const Plan& p, char* ws, hipStream_t s, int* check_slot) {
  int rc;
  const pa_cache_desc* cache = c.cache;
  if (check_on()) {
    pa::CheckArgs ck{};
    ck.block_tables = c.block_tables;
    ck.seq_lens = c.seq_lens;
    ck.qsl = c.qsl;
    ck.num_seqs = c.B;
    ck.max_blocks = c.MB;
    ck.num_blocks = cache->num_blocks;
    ck.num_q_tokens = c.T;
    ck.window = c.window;
    ck.max_q_len = c.max_q_len;
    rc = run_check(ck, s, check_slot);
    if (rc) return rc;
  }

  const float scale_log2 = c.scale * 1.4426950408889634f;
  auto run_decode = [&](hipStream_t s) -> int {
    int rc;
  if (p.run_decode) {
      pa::DecodeArgs d{};
      d.q = c.q;
      d.k_cache = c.k_cache;
      d.v_cache = c.v_cache;
      d.block_tables = c.block_tables;
      d.seq_lens = c.seq_lens;
      d.qsl = c.qsl;
      d.out = c.out;
      d.part_o = p.max_splits > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
      d.part_ml = p.max_splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
      d.num_seqs = c.B;
      d.num_rows = p.rows;
      d.per_token = p.per_token;
      d.qmax = p.qmax;
      d.num_q_heads = c.Hq;
      d.num_kv_heads = cache->num_kv_heads;
      d.group = p.group;
      d.heads_per_wg = p.heads_per_wg;
      d.max_blocks = c.MB;
      d.split = p.split;
      d.max_splits = p.max_splits;
      d.stream_wgs = 0;
      if (p.stream) {
        rc = stream_wgs(p, cache->num_kv_heads, d.stream_wgs);
        if (rc) return rc;
      } else if (cache->dtype == PA_DTYPE_BF16) {
        // split-mode bf16 decode: two-KV-head workgroups (one wave per SIMD) when the grid of
        // four-head ones (two resident per CU) makes at least two chip-wide rounds
        int cus = 0;
        rc = chip_cus(cus);
        if (rc) return rc;
        const int64_t units4 = (int64_t)((cache->num_kv_heads + 3) / 4) * p.max_splits * p.rows;
        d.pair_wgs = units4 >= 4 * (int64_t)cus;
      }
      d.window = c.window;
      d.scale_log2 = scale_log2;
      d.k_scale = cache->k_scale;
      d.v_scale = cache->v_scale;
      hipError_t e = timed("decode_split", s, [&] {
        return p.i8 ? pa::launch_decode_split_i8(d, p.head_dim, s) : pa::launch_decode_split(d, p.head_dim, p.bf16, s);
      });
      if (e != hipSuccess) return device_fail(e, "decode split launch");
      if (p.max_splits > 1) {
        e = timed("decode_merge", s, [&] { return pa::launch_decode_merge(d, p.head_dim, p.bf16, s); });
        if (e != hipSuccess) return device_fail(e, "decode merge launch");
      }
    }
    return PA_OK;
  };
  auto run_tiles = [&](hipStream_t s) -> int {
  if (p.run_tiles) {
      pa::TileArgs t{};
      t.q = c.q;
      t.k_cache = c.k_cache;
      t.v_cache = c.v_cache;
      t.block_tables = c.block_tables;
      t.seq_lens = c.seq_lens;
      t.qsl = c.qsl;
      t.out = c.out;
      t.num_seqs = c.B;
      t.min_q = p.qmax + 1;
      t.num_slots = p.num_slots;
      t.num_q_heads = c.Hq;
      t.num_kv_heads = cache->num_kv_heads;
      t.group = p.group;
      t.pos_per_tile = p.pos_per_tile;
      t.max_blocks = c.MB;
      t.window = c.window;
      t.scale_log2 = scale_log2;
      t.k_scale = cache->k_scale;
      t.v_scale = cache->v_scale;
      const hipError_t e = timed("prefill_tile", s, [&] { return pa::launch_prefill_tile(t, p.head_dim, p.i8, s); });
      if (e != hipSuccess) return device_fail(e, "prefill tile launch");
    }
    return PA_OK;
  };
  if (p.run_decode && p.run_tiles && !check_slot) {
    // decode rows on the device's side stream, concurrently with the tiles on the caller's stream
    // (the no-allocation entry point, which passes check_slot, creates no stream and runs both
    // passes on the caller's stream)
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    rc = side_stream(side, fork, join);
    if (rc) return rc;
    std::lock_guard<std::mutex> lk(g_side_mu);
    hipError_t e = hipEventRecord(fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
    if (e != hipSuccess) return device_fail(e, "fork to the side stream");
    rc = run_tiles(s);
    if (rc) return rc;
    rc = run_decode(side);
    if (rc) return rc;
    e = hipEventRecord(join, side);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, join, 0);
    if (e != hipSuccess) return device_fail(e, "join from the side stream");
    return PA_OK;
  }
  if (p.run_decode) {
    rc = run_decode(s);
    if (rc) return rc;
  }
  if (p.run_tiles) return run_tiles(s);
  return PA_OK;
}

}  // namespace

// ---- the no-allocation entry point's scratch: a fixed array in each device's memory ----
// In host code `scratch` is only a stand-in for the symbol: kernels and copies get the address
// that hipGetSymbolAddress returns for the current device (each device holds its own copy).
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr size_t kScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCheck = 256;              // first bytes: the check-mode result slot
static_assert(kScratchBytes > kScratchCheck, "scratch holds the check slot and a workspace");

std::mutex g_scratch_mu;
std::unordered_map<int, char*> g_scratch;          // device -> address of its scratch array

int scratch_address(char*& ptr) {
  int dev = 0;
  int rc = get_device(dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return device_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    it = g_scratch.emplace(dev, static_cast<char*>(p)).first;
  }
  ptr = it->second;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_last_error(void) { return g_err.c_str(); }

void pa_set_check(int on) { g_check.store(on ? 1 : 0); }

void pa_release(void) {   // best effort: errors here have nowhere to go
  int cur = 0;
  (void)hipGetDevice(&cur);
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    for (auto& kv : g_ws) {
      (void)hipSetDevice(kv.first.first);
      (void)hipDeviceSynchronize();
      if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    }
    g_ws.clear();
  }
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    for (auto& kv : g_dev) {
      (void)hipSetDevice(kv.first);
      (void)hipDeviceSynchronize();
      if (kv.second.check) (void)hipFree(kv.second.check);
      kv.second = DevState{};
    }
    g_dev.clear();
  }
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    for (auto& kv : g_side) {
      (void)hipSetDevice(kv.first);
      if (kv.second.s) (void)hipStreamSynchronize(kv.second.s);
      if (kv.second.fork) (void)hipEventDestroy(kv.second.fork);
      if (kv.second.join) (void)hipEventDestroy(kv.second.join);
      if (kv.second.s) (void)hipStreamDestroy(kv.second.s);
    }
    g_side.clear();
  }
  (void)hipSetDevice(cur);
}

int pa_append_kv(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens, void* k_cache,
                 void* v_cache, const pa_cache_desc* cache, void* stream) {
  g_err.clear();
  int rc = validate_desc(cache);
  if (rc) return rc;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (k_cache == v_cache) return fail(PA_ERR_INVALID_ARG, "k_cache and v_cache must differ");
  if (misaligned(k) || misaligned(v) || misaligned(k_cache) || misaligned(v_cache))
    return fail(PA_ERR_INVALID_ARG, "k, v and the caches must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t esz = cache->dtype == PA_DTYPE_F32 ? 4 : 2;         // input rows (bf16 for int8 caches)
  if (check_on()) {
    pa::CheckArgs c{};
    c.slot_mapping = slot_mapping;
    c.num_tokens = num_tokens;
    c.num_slots = (int64_t)cache->num_blocks * PA_BLOCK_SIZE;
    rc = run_check(c, s);
    if (rc) return rc;
  }
  pa::AppendArgs a{k, v, slot_mapping, k_cache, v_cache, num_tokens, (int64_t)cache->num_kv_heads * cache->head_dim * esz,
                   cache->k_scale, cache->v_scale};
  hipError_t e = timed("append", s, [&] { return pa::launch_append(a, s); });
  if (e != hipSuccess) return device_fail(e, "append launch");
  return PA_OK;
}

size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_q_tokens, int32_t max_blocks_per_seq,
                                   int32_t num_q_heads, const pa_cache_desc* cache) {
  Plan p;
  std::string keep = g_err;
  if (make_plan(num_seqs, num_q_tokens, max_blocks_per_seq, num_q_heads, cache, pa::kNoWindow, 0, p, true) != PA_OK) {
    g_err = keep;
    return 0;
  }
  return p.total > 0 ? p.total : 256;
}

int pa_attention_ex(const void* q, int32_t num_q_tokens, int32_t num_q_heads, const void* k_cache,
                    const void* v_cache, const pa_cache_desc* cache, const int32_t* block_tables, int32_t num_seqs,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, const int32_t* query_start_loc, float scale,
                    void* out, void* workspace, size_t workspace_bytes, const pa_attention_opts* opts,
                    void* stream) {
  g_err.clear();
  const Call given{q, num_q_tokens, num_q_heads, k_cache, v_cache, cache, block_tables, num_seqs,
                   max_blocks_per_seq, seq_lens, query_start_loc, scale, out, 0, 0};
  Call c;
  Plan p;
  int rc = prepare(given, opts, c, p);
  if (rc) return rc;
  if (misaligned(workspace)) return fail(PA_ERR_INVALID_ARG, "q, the caches, out and the workspace must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.total == 0) return launch_call(c, p, nullptr, s, nullptr);
  if (workspace) {
    if (workspace_bytes < p.total)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, p.total);
    return launch_call(c, p, static_cast<char*>(workspace), s, nullptr);
  }
  // library-owned buffer of this (device, stream), held locked until the kernels are queued
  int dev = 0;
  rc = get_device(dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  StreamWs& ws = g_ws[{dev, reinterpret_cast<uintptr_t>(s)}];
  if (ws.bytes < p.total) {
    if (ws.ptr) {
      hipError_t e = hipStreamSynchronize(s);               // the stream's earlier calls may still read it
      if (e == hipSuccess) e = hipFree(ws.ptr);
      ws = StreamWs{};
      if (e != hipSuccess) return device_fail(e, "releasing the old workspace");
    }
    hipError_t e = hipMalloc(&ws.ptr, p.total);
    if (e != hipSuccess) {
      ws = StreamWs{};
      return device_fail(e, "hipMalloc(workspace)");
    }
    ws.bytes = p.total;
  }
  return launch_call(c, p, static_cast<char*>(ws.ptr), s, nullptr);
}

int pa_attention(const void* q, int32_t num_q_tokens, int32_t num_q_heads, const void* k_cache, const void* v_cache,
                 const pa_cache_desc* cache, const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                 const int32_t* seq_lens, const int32_t* query_start_loc, float scale, void* out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return pa_attention_ex(q, num_q_tokens, num_q_heads, k_cache, v_cache, cache, block_tables, num_seqs,
                         max_blocks_per_seq, seq_lens, query_start_loc, scale, out, workspace, workspace_bytes,
                         nullptr, stream);
}

int pa_attention_noalloc(const void* q, int32_t num_q_tokens, int32_t num_q_heads, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* cache, const int32_t* block_tables,
                         int32_t num_seqs, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         const int32_t* query_start_loc, float scale, void* out, const pa_attention_opts* opts,
                         void* stream) {
  g_err.clear();
  const Call given{q, num_q_tokens, num_q_heads, k_cache, v_cache, cache, block_tables, num_seqs,
                   max_blocks_per_seq, seq_lens, query_start_loc, scale, out, 0, 0};
  Call c;
  Plan p;
  int rc = prepare(given, opts, c, p);
  if (rc) return rc;
  if (p.total > kScratchBytes - kScratchCheck)
    return fail(PA_ERR_WORKSPACE, "this batch needs %zu bytes of scratch; the no-allocation entry point holds %zu",
                p.total, kScratchBytes - kScratchCheck);
  char* base = nullptr;
  rc = scratch_address(base);
  if (rc) return rc;
  return launch_call(c, p, base + kScratchCheck, reinterpret_cast<hipStream_t>(stream), reinterpret_cast<int*>(base));
}

int pa_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  g_timing = on != 0;
  return PA_OK;
}

int pa_timing_read(const char* name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  for (auto& t : g_pending) {
    hipError_t e = hipEventSynchronize(t.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.a, t.b);
    if (e != hipSuccess) return device_fail(e, "timing event");
    auto& acc = g_t_acc[t.name];
    acc.first += ms;
    acc.second += 1;
    g_event_pool.push_back(t.a);
    g_event_pool.push_back(t.b);
  }
  g_pending.clear();
  auto it = g_t_acc.find(name ? name : "");
  if (total_ms) *total_ms = it == g_t_acc.end() ? 0.0 : it->second.first;
  if (launches) *launches = it == g_t_acc.end() ? 0 : it->second.second;
  return PA_OK;
}

void pa_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  for (auto& t : g_pending) {
    (void)hipEventSynchronize(t.b);                          // best effort: the events are recycled
    g_event_pool.push_back(t.a);
    g_event_pool.push_back(t.b);
  }
  g_pending.clear();
  g_t_acc.clear();
}

}  // extern "C"
