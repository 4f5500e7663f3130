/*
 * pa_oracle.c -- plain, slow CPU reference for causal attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no source with the HIP kernels and links no HIP.
 *
 * Sources (four web pages on paged attention):
 *   P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576)
 *   P3  prefill/decode article on the page titled "企业官网建设流程全解析" (hotelren.com/news/6181127)
 *   P4  "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill)
 *
 * What it computes is the plain definition, written out:
 *   append     -- each new token's K and V row is copied to the cache slot given for it
 *                 (P3 §2.3: only K and V are cached; P1 §2.2: rows are written by page index).
 *   attention  -- for request b, query row r sits at absolute position p = ctx + r, where
 *                 ctx = seq_len - q_len (P4 "把长输入切成块": a chunk reads the earlier KV, then its
 *                 own).  Its keys are gathered through the block table (P1 §3.3: page-table lookup,
 *                 then the address), scores are scale * q.k for every key, keys j > p are set to
 *                 -inf (P3 §1.1, §2.1: position i depends only on 0..i, the upper triangle is masked
 *                 before the softmax), a row softmax follows and the weights multiply V
 *                 (P3 §3.1, §5.1: softmax(q K^T) V over all cached keys).  With a sliding window
 *                 W > 0, keys j < p - W + 1 are also set to -inf (P3 §6.3, P2 §5.2: keep only the
 *                 most recent W tokens' K/V); keys that no row can see are not gathered.
 *   8-bit cache -- P2 §4.3 and §5.4 (INT8 KV halves memory and bandwidth; calibrate per channel):
 *                 the cache holds int8 codes with one fp32 scale per (KV head, channel).  Append
 *                 quantises each element of the bf16 input x with its channel's scale s:
 *                 code = x / s rounded to fp32, then to the nearest integer (ties to even), clamped
 *                 to [-127, 127]; NaN gives 0.  Attention reads code * s (exact in double) and is
 *                 otherwise the computation above.
 * Precision: inputs are widened exactly to double (bf16: bits << 16), every sum is in double,
 * and the result is rounded once to the output dtype (bf16: nearest, ties to even).
 *
 * Parity: pinned by the tests against a library dense causal softmax on tiny inputs, closed
 * forms (constant V, zero K, single visible key), argmax probes, block-permutation invariance,
 * chunked == one-shot and decode == last prefill row; the window by a library softmax over each
 * row's key slice, W >= context == no window, W = 1 == own V row, and a dominant key one step
 * outside / at the window's edge; the int8 path by hand-computed codes (exact multiples, ties,
 * clamps, NaN), the fp32 quotient deciding the rounding, bitwise equality with the fp32 path over
 * a dequantised cache, a library softmax over dequantised values and a dequantised argmax probe.
 * No page prints attention output values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 16

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2 };

static void set_err(char* err, int err_len, const char* msg) {
  if (err && err_len > 0) {
    strncpy(err, msg, (size_t)err_len - 1);
    err[err_len - 1] = 0;
  }
}

static double load_elem(const void* base, size_t idx, int dtype) {
  if (dtype == OR_F32) return (double)((const float*)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to bfloat16, nearest with ties to even, in one step from the exact value. */
uint16_t pa_oracle_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (isinf(ax)) return sign | 0x7F80;
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e);                 /* ax = m * 2^e, m in [0.5, 1) */
  int qe = e - 8;                /* bf16 keeps 8 significant bits */
  if (qe < -133) qe = -133;      /* subnormal spacing 2^-133 */
  double r = nearbyint(ldexp(ax, -qe)); /* default rounding mode: ties to even */
  double y = ldexp(r, qe);
  float f = (float)y;            /* exact (8 significant bits) unless it overflows to inf */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

static void store_elem(void* base, size_t idx, int dtype, double v) {
  if (dtype == OR_F32) ((float*)base)[idx] = (float)v;
  else ((uint16_t*)base)[idx] = pa_oracle_f64_to_bf16(v);
}

/* ---------------------------------------------------------------------------------------- */
/* append                                                                                    */
/* ---------------------------------------------------------------------------------------- */
/* Slots must lie in the pool and be distinct (negative = skip).  Returns 0 or an error code. */
static int check_slots(const int32_t* slot_mapping, int32_t num_tokens, int64_t nslots, char* err, int err_len) {
  unsigned char* seen = (unsigned char*)calloc((size_t)nslots, 1);
  if (!seen) { set_err(err, err_len, "oom"); return 1; }
  for (int32_t i = 0; i < num_tokens; ++i) {
    int32_t s = slot_mapping[i];
    if (s < 0) continue;
    if ((int64_t)s >= nslots) {
      char m[128];
      snprintf(m, sizeof m, "slot %d of token %d is outside the pool", s, i);
      set_err(err, err_len, m);
      free(seen);
      return 2;
    }
    if (seen[s]) {
      char m[128];
      snprintf(m, sizeof m, "slot %d written twice (token %d)", s, i);
      set_err(err, err_len, m);
      free(seen);
      return 3;
    }
    seen[s] = 1;
  }
  free(seen);
  return 0;
}

/* int8 code of x under scale s (see the header): fp32 quotient, nearest-even, clamp, NaN -> 0. */
static int8_t quantize(float x, float s) {
  float r = x / s;                 /* one IEEE single-precision division */
  if (r != r) return 0;
  r = rintf(r);                    /* default rounding mode: nearest, ties to even */
  if (r > 127.f) r = 127.f;
  if (r < -127.f) r = -127.f;
  return (int8_t)r;
}

int pa_oracle_quantize(float x, float s) { return quantize(x, s); }

int pa_oracle_append_i8(const uint16_t* k, const uint16_t* v, const int32_t* slot_mapping, int32_t num_tokens,
                        int8_t* k_cache, int8_t* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, const float* k_scale, const float* v_scale, char* err, int32_t err_len) {
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1 || head_dim < 1 || !k_scale || !v_scale) {
    set_err(err, err_len, "bad sizes");
    return 1;
  }
  int rc = check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * ORACLE_BLOCK, err, err_len);
  if (rc) return rc;
  const size_t row = (size_t)num_kv_heads * (size_t)head_dim;
  for (int32_t i = 0; i < num_tokens; ++i) {
    int32_t s = slot_mapping[i];
    if (s < 0) continue;
    for (size_t c = 0; c < row; ++c) {
      k_cache[(size_t)s * row + c] = quantize((float)load_elem(k, (size_t)i * row + c, OR_BF16), k_scale[c]);
      v_cache[(size_t)s * row + c] = quantize((float)load_elem(v, (size_t)i * row + c, OR_BF16), v_scale[c]);
    }
  }
  return 0;
}

int pa_oracle_append(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                     void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                     int32_t head_dim, int32_t esz, char* err, int32_t err_len) {
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1 || head_dim < 1 || (esz != 2 && esz != 4)) {
    set_err(err, err_len, "bad sizes");
    return 1;
  }
  int64_t nslots = (int64_t)num_blocks * ORACLE_BLOCK;
  size_t row = (size_t)num_kv_heads * (size_t)head_dim * (size_t)esz;
  int rc = check_slots(slot_mapping, num_tokens, nslots, err, err_len);
  if (rc) return rc;
  for (int32_t i = 0; i < num_tokens; ++i) {
    int32_t s = slot_mapping[i];
    if (s < 0) continue;                       /* padding token: nothing to write */
    memcpy((char*)k_cache + (size_t)s * row, (const char*)k + (size_t)i * row, row);
    memcpy((char*)v_cache + (size_t)s * row, (const char*)v + (size_t)i * row, row);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* attention                                                                                 */
/* ---------------------------------------------------------------------------------------- */
typedef struct {
  /* shared, read-only */
  const void* q;
  int dtype, Hq, Hkv, d;
  int G;
  int window;         /* > 0: row p sees only keys p - window + 1 .. p */
  double scale;
  const double* Kb;   /* gathered keys   [s][Hkv][d] */
  const double* Vb;   /* gathered values [s][Hkv][d] */
  int s, ctx, q0;
  const int32_t* rows; /* request-local row indices to compute */
  int nrows;
  void* out;
  double* out_f64;
  int nthreads;
  int tid;
} job_t;

static void row_head(const job_t* J, int r, int h) {
  const int d = J->d, s = J->s;
  const int g = h / J->G;                   /* contiguous groups of query heads share a KV head */
  const int p = J->ctx + r;                 /* absolute position of this query row */
  const size_t t = (size_t)(J->q0 + r);
  double* x = (double*)malloc(sizeof(double) * (size_t)s);
  double* acc = (double*)calloc((size_t)d, sizeof(double));
  double* qv = (double*)malloc(sizeof(double) * (size_t)d);
  for (int c = 0; c < d; ++c) qv[c] = load_elem(J->q, (t * J->Hq + h) * d + c, J->dtype);
  /* scores for every key */
  for (int j = 0; j < s; ++j) {
    const double* kr = J->Kb + ((size_t)j * J->Hkv + g) * d;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += qv[c] * kr[c];
    x[j] = J->scale * dot;
  }
  /* explicit causal mask, and the sliding-window lower bound when a window is set */
  for (int j = 0; j < s; ++j)
    if (j > p) x[j] = -INFINITY;
  if (J->window > 0)
    for (int j = 0; j < s; ++j)
      if (j < p - J->window + 1) x[j] = -INFINITY;
  double m = -INFINITY;
  for (int j = 0; j < s; ++j)
    if (x[j] > m) m = x[j];
  double l = 0.0;
  for (int j = 0; j < s; ++j) {
    double e = (x[j] == -INFINITY) ? 0.0 : exp(x[j] - m);
    if (e == 0.0) continue;
    l += e;
    const double* vr = J->Vb + ((size_t)j * J->Hkv + g) * d;
    for (int c = 0; c < d; ++c) acc[c] += e * vr[c];
  }
  for (int c = 0; c < d; ++c) {
    double o = acc[c] / l;
    size_t idx = (t * J->Hq + h) * d + c;
    if (J->out) store_elem(J->out, idx, J->dtype, o);
    if (J->out_f64) J->out_f64[idx] = o;
  }
  free(x);
  free(acc);
  free(qv);
}

static void* worker(void* arg) {
  const job_t* J = (const job_t*)arg;
  int64_t n = (int64_t)J->nrows * J->Hq;
  for (int64_t i = J->tid; i < n; i += J->nthreads) row_head(J, J->rows[i / J->Hq], (int)(i % J->Hq));
  return NULL;
}

typedef struct {
  const void* kc;
  const void* vc;
  int dtype, Hkv, d;          /* dtype of the cache elements */
  const float* k_scale;       /* [Hkv][d], int8 caches only */
  const float* v_scale;
  const int32_t* table;
  double* Kb;
  double* Vb;
  int s, j0, tid, nthreads;   /* gather keys j0 .. s-1 (earlier ones are never visible) */
} gather_t;

static void* gather_worker(void* arg) {
  const gather_t* Gt = (const gather_t*)arg;
  const size_t row = (size_t)Gt->Hkv * Gt->d;
  for (int j = Gt->j0 + Gt->tid; j < Gt->s; j += Gt->nthreads) {
    const int blk = Gt->table[j / ORACLE_BLOCK];
    const size_t src = ((size_t)blk * ORACLE_BLOCK + (size_t)(j % ORACLE_BLOCK)) * row;
    for (size_t c = 0; c < row; ++c) {
      if (Gt->dtype == OR_I8) {             /* dequantise: code * scale of (head, channel) c */
        Gt->Kb[(size_t)j * row + c] = (double)((const int8_t*)Gt->kc)[src + c] * (double)Gt->k_scale[c];
        Gt->Vb[(size_t)j * row + c] = (double)((const int8_t*)Gt->vc)[src + c] * (double)Gt->v_scale[c];
      } else {
        Gt->Kb[(size_t)j * row + c] = load_elem(Gt->kc, src + c, Gt->dtype);
        Gt->Vb[(size_t)j * row + c] = load_elem(Gt->vc, src + c, Gt->dtype);
      }
    }
  }
  return NULL;
}

int pa_oracle_attention(const void* q, int32_t num_tokens, int32_t num_q_heads,
                        const void* k_cache, const void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, int32_t dtype, int32_t cache_dtype, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables, int32_t num_seqs,
                        int32_t max_blocks, const int32_t* seq_lens, const int32_t* query_start_loc,
                        double scale, int32_t window, const int32_t* rows, int32_t num_rows, void* out,
                        double* out_f64, int32_t num_threads, char* err, int32_t err_len) {
  char m[256];
  if (num_seqs < 1 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      num_q_heads % num_kv_heads != 0 || (dtype != OR_F32 && dtype != OR_BF16) || max_blocks < 1 ||
      window < 0 || (cache_dtype != dtype && !(cache_dtype == OR_I8 && dtype == OR_BF16)) ||
      (cache_dtype == OR_I8 && (!k_scale || !v_scale))) {
    set_err(err, err_len, "bad sizes");
    return 1;
  }
  if (query_start_loc[0] != 0 || query_start_loc[num_seqs] != num_tokens) {
    set_err(err, err_len, "query_start_loc must start at 0 and end at num_tokens");
    return 1;
  }
  for (int b = 0; b < num_seqs; ++b) {
    int ql = query_start_loc[b + 1] - query_start_loc[b];
    int s = seq_lens[b];
    if (ql < 1 || s < ql || s > max_blocks * ORACLE_BLOCK) {
      snprintf(m, sizeof m, "request %d: need 1 <= q_len (%d) <= seq_len (%d) <= %d", b, ql, s,
               max_blocks * ORACLE_BLOCK);
      set_err(err, err_len, m);
      return 1;
    }
    /* with a window, blocks wholly before the first row's window are never read */
    int first = 0;
    if (window > 0 && s - ql - window + 1 > 0) first = (s - ql - window + 1) / ORACLE_BLOCK;
    for (int j = first; j < (s + ORACLE_BLOCK - 1) / ORACLE_BLOCK; ++j) {
      int blk = block_tables[(size_t)b * max_blocks + j];
      if (blk < 0 || blk >= num_blocks) {
        snprintf(m, sizeof m, "request %d: block table entry %d = %d outside the pool", b, j, blk);
        set_err(err, err_len, m);
        return 2;
      }
    }
  }
  if (num_threads < 1) num_threads = 1;
  /* which token rows to compute */
  int32_t* want = (int32_t*)calloc((size_t)(num_tokens > 0 ? num_tokens : 1), sizeof(int32_t));
  if (rows) {
    for (int i = 0; i < num_rows; ++i) {
      if (rows[i] < 0 || rows[i] >= num_tokens) {
        set_err(err, err_len, "row index out of range");
        free(want);
        return 1;
      }
      want[rows[i]] = 1;
    }
  } else {
    for (int i = 0; i < num_tokens; ++i) want[i] = 1;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)num_threads);
  int rc = 0;
  for (int b = 0; b < num_seqs && rc == 0; ++b) {
    const int q0 = query_start_loc[b], ql = query_start_loc[b + 1] - q0, s = seq_lens[b];
    int nr = 0;
    for (int r = 0; r < ql; ++r) nr += want[q0 + r];
    if (nr == 0) continue;
    int32_t* rl = (int32_t*)malloc(sizeof(int32_t) * (size_t)nr);
    nr = 0;
    for (int r = 0; r < ql; ++r)
      if (want[q0 + r]) rl[nr++] = r;
    /* explicit gather of this request's keys and values through its block table */
    const size_t row = (size_t)num_kv_heads * head_dim;
    const int j0 = (window > 0 && s - ql - window + 1 > 0) ? (s - ql - window + 1) : 0;
    double* Kb = (double*)calloc((size_t)s * row, sizeof(double));
    double* Vb = (double*)calloc((size_t)s * row, sizeof(double));
    if (!Kb || !Vb) {
      set_err(err, err_len, "oom");
      free(Kb); free(Vb); free(rl);
      rc = 4;
      break;
    }
    gather_t* gt = (gather_t*)malloc(sizeof(gather_t) * (size_t)num_threads);
    for (int i = 0; i < num_threads; ++i) {
      gather_t g0 = {k_cache, v_cache, cache_dtype, num_kv_heads, head_dim, k_scale, v_scale,
                     block_tables + (size_t)b * max_blocks, Kb, Vb, s, j0, i, num_threads};
      gt[i] = g0;
      pthread_create(&th[i], NULL, gather_worker, &gt[i]);
    }
    for (int i = 0; i < num_threads; ++i) pthread_join(th[i], NULL);
    free(gt);
    job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)num_threads);
    for (int i = 0; i < num_threads; ++i) {
      job_t jb = {q, dtype, num_q_heads, num_kv_heads, head_dim, num_q_heads / num_kv_heads, window, scale,
                  Kb, Vb, s, s - ql, q0, rl, nr, out, out_f64, num_threads, i};
      jobs[i] = jb;
      pthread_create(&th[i], NULL, worker, &jobs[i]);
    }
    for (int i = 0; i < num_threads; ++i) pthread_join(th[i], NULL);
    free(jobs);
    free(Kb);
    free(Vb);
    free(rl);
  }
  free(th);
  free(want);
  return rc;
}
