// pa_rows.h -- which keys a decode-pass row sees: shared by the split kernels and the merge.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

// Resolve a row slot to (request, token, causal keys).  Returns false if the slot is not a
// row of this pass (bf16 and int8 requests with q_len != 1 go to the tile kernel).
__device__ __forceinline__ bool resolve_row(const DecodeArgs& a, int row, int& b, int& t, int& n_keys) {
  if (a.per_token) {
    t = row;
    int lo = 0, hi = a.num_seqs;                       // qsl[lo] <= t < qsl[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.qsl[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
  } else {
    b = row;
    if (a.qsl[b + 1] - a.qsl[b] != 1) return false;
    t = a.qsl[b];
  }
  const int q0 = a.qsl[b];
  const int ql = a.qsl[b + 1] - q0;
  n_keys = a.seq_lens[b] - ql + (t - q0) + 1;          // keys 0 .. position of this row
  return true;
}

// First key a row with `n_keys` causal keys sees (a sliding window drops the older ones), and the
// block-aligned key where its splits begin.  Every kernel of the pass derives its ranges from these.
__device__ __forceinline__ int first_visible(const DecodeArgs& a, int n_keys) { return max(0, n_keys - a.window); }
__device__ __forceinline__ int split_origin(const DecodeArgs& a, int n_keys) {
  return first_visible(a, n_keys) & ~(kBlock - 1);
}

}  // namespace pa
