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

// Index of the split partial of (row, position r, split, query head h).
__device__ __forceinline__ int64_t partial_index(const DecodeArgs& a, int row, int r, int split, int h) {
  return (((int64_t)row * a.qmax + r) * a.max_splits + split) * a.num_q_heads + h;
}

}  // namespace pa
