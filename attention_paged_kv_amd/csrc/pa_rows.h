// pa_rows.h -- which keys a decode-pass row sees: shared by the split kernels and the merge.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

// Resolve a row slot to (request, first token, causal keys of its last position, positions).
// Per-token rows (fp32) are one position each.  Request rows carry q_len <= a.qmax positions
// (decode, or a few tokens to verify); others are not rows of this pass (the tile kernel's).
__device__ __forceinline__ bool resolve_row(const DecodeArgs& a, int row, int& b, int& t, int& n_keys, int& ql) {
  if (a.per_token) {
    t = row;
    int lo = 0, hi = a.num_seqs;                       // qsl[lo] <= t < qsl[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.qsl[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
    const int q0 = a.qsl[b];
    n_keys = a.seq_lens[b] - (a.qsl[b + 1] - q0) + (t - q0) + 1;   // keys 0 .. position of this token
    ql = 1;
    return true;
  }
  b = row;
  ql = a.qsl[b + 1] - a.qsl[b];
  if (ql < 1 || ql > a.qmax) return false;
  t = a.qsl[b];
  n_keys = a.seq_lens[b];                              // keys of the last position
  return true;
}

// First key a position with `n` causal keys sees (a sliding window drops the older ones), and the
// block-aligned key where a row's splits begin: that of its first position, whose window starts
// earliest.  Every kernel of the pass derives its ranges from these.
__device__ __forceinline__ int first_visible(const DecodeArgs& a, int n) { return max(0, n - a.window); }
__device__ __forceinline__ int split_origin(const DecodeArgs& a, int n_keys, int ql) {
  return first_visible(a, n_keys - ql + 1) & ~(kBlock - 1);
}

// ---- stream mode (decode over a bf16 or int8 cache) ----
// The 16-key blocks that the rows' passes cover, concatenated in row order, are dealt out in equal
// runs of L blocks to stream_wgs workgroups per head group (bf16: two KV heads; int8: four KV heads
// and one column group).  A run may end one row and begin the
// next; each (row, run) piece is a partial softmax of the row, like a split, and a row's pieces
// are merged as splits are.  Every workgroup reads the same number of blocks, so the launch has
// no tail of workgroups still running while the rest of the chip idles.

// Blocks a row's pass covers: from the block holding the oldest key its first position sees to
// the block holding its last key; 0 for rows that are not on this pass.
__device__ __forceinline__ int row_blocks(const DecodeArgs& a, int row) {
  int b, t, n_keys, ql;
  if (row >= a.num_rows || !resolve_row(a, row, b, t, n_keys, ql) || n_keys < 1) return 0;
  return (n_keys + kBlock - 1) / kBlock - first_visible(a, n_keys - ql + 1) / kBlock;
}

// Blocks of all rows (the wave's lanes take 64 rows at a time); for row `want` also the blocks
// before it (pre) and its own (nb).
__device__ __forceinline__ int stream_scan(const DecodeArgs& a, int want, int& pre, int& nb) {
  const int lane = threadIdx.x & (kWave - 1);
  int base = 0;
  pre = 0;
  nb = 0;
  for (int c0 = 0; c0 < a.num_rows; c0 += kWave) {
    const int v = row_blocks(a, c0 + lane);
    const int incl = wave_incl_scan(v);
    if (want >= c0 && want < c0 + kWave) {
      pre = base + __builtin_amdgcn_readlane(incl - v, want - c0);
      nb = __builtin_amdgcn_readlane(v, want - c0);
    }
    base += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return base;
}

// Blocks per run, given the total: an equal share, but at least `split` keys.
__device__ __forceinline__ int stream_run(const DecodeArgs& a, int tot) {
  return max((int)(((int64_t)tot + a.stream_wgs - 1) / a.stream_wgs), a.split / kBlock);
}

// Pieces of a row whose blocks are [pre, pre + nb) of the concatenation: the runs it meets.
__device__ __forceinline__ int stream_pieces(int pre, int nb, int run) {
  return nb < 1 ? 0 : (pre + nb - 1) / run - pre / run + 1;
}

// Walks the concatenation: the row holding block g, for g increasing.
struct BlockCursor {
  int c0 = -kWave, base = 0, tot = 0, incl = 0, v = 0;
  __device__ bool seek(const DecodeArgs& a, int g, int& row, int& pre, int& nb) {
    while (c0 < 0 || g >= base + tot) {
      if (c0 + kWave >= a.num_rows) return false;        // g is past the last row
      if (c0 >= 0) base += tot;
      c0 += kWave;
      v = row_blocks(a, c0 + (int)(threadIdx.x & (kWave - 1)));
      incl = wave_incl_scan(v);
      tot = __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    const int j = __popcll(__ballot(incl <= g - base));   // rows wholly before block g
    row = c0 + j;
    pre = base + __builtin_amdgcn_readlane(incl - v, j);
    nb = __builtin_amdgcn_readlane(v, j);
    return true;
  }
};

// Lane i (lanes below count) loads block id p[i] and waits for it, in inline assembly: a load the
// compiler sees inside a block loop makes it wait for every outstanding copy on every block after.
__device__ __forceinline__ int load_ids_sync(const int32_t* p, int count) {
  int v = 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t* q = p + lane;
  if (lane < count) asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(q) : "memory");
  return v;
}

// Index of the split partial of (row, position r, split, query head h).
__device__ __forceinline__ int64_t partial_index(const DecodeArgs& a, int row, int r, int split, int h) {
  return (((int64_t)row * a.qmax + r) * a.max_splits + split) * a.num_q_heads + h;
}

}  // namespace pa
