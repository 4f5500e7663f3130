// pa_decode.hip -- split-KV attention for single query rows, and the cross-split merge.
//
// A decode step reads every cached key and value of its request once (P3 §3.1-3.2, §6.3): the
// pass is bound by HBM bandwidth, not arithmetic.  Work unit = (query row, KV head, split of
// `split` keys).  A workgroup loads each K/V row of its KV head once and uses it for all the
// query heads of the group it owns (grouped-query sharing, P3 §2.3).  Inside the workgroup every
// 16-lane row group keeps its own running max / sum / accumulator (online softmax over 16-key
// blocks); the row groups and the four waves are merged at the end, and splits of one row are
// merged by a second kernel with the same log-sum-exp rule:
//   m = max_s m_s,  l = sum_s 2^(m_s - m) l_s,  o = sum_s 2^(m_s - m) o_s / l
// (scores are kept in log2 units: x * scale * log2 e).  The pages do not describe how partial
// softmaxes are combined; this is the exact decomposition of the row softmax of P3 §3.1.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <bool BF16>
struct Io;

template <>
struct Io<true> {
  static constexpr int kEsz = 2;
  static constexpr int kEpl = 8;   // elements per 16-byte load
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  __device__ static void store(void* base, int64_t idx, float v) {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
  }
};

template <>
struct Io<false> {
  static constexpr int kEsz = 4;
  static constexpr int kEpl = 4;
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static void store(void* base, int64_t idx, float v) { reinterpret_cast<float*>(base)[idx] = v; }
};

// Resolve a row slot to (request, token, visible keys).  Returns false if the slot is not a
// row of this pass (bf16 requests with q_len != 1 go to the tile kernel).
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

__device__ __forceinline__ float wave_max_over_groups(float v, int lpr) {
  for (int o = lpr; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_over_groups(float v, int lpr) {
  for (int o = lpr; o < kWave; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

template <int D, int GT, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  using IO = Io<BF16>;
  constexpr int EPL = IO::kEpl;
  constexpr int LPR = D * IO::kEsz / 16;     // lanes per K/V row
  constexpr int RPL = kWave / LPR;           // rows per wave-wide load
  constexpr int LPB = kBlock / RPL;          // loads per 16-key block
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row width");

  __shared__ float sm_m[4][GT];
  __shared__ float sm_l[4][GT];
  __shared__ float sm_o[4][GT][D];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int rg = lane / LPR;                 // row group within the wave
  const int cl = lane % LPR;                 // which 16-byte piece of the row

  const int nz = a.num_kv_heads * (a.group / GT);
  int u = blockIdx.x;
  const int z = u % nz;
  u /= nz;
  const int split = u % a.max_splits;
  const int row = u / a.max_splits;
  if (row >= a.num_rows) return;
  int b, t, n_keys;
  if (!resolve_row(a, row, b, t, n_keys)) return;
  const int k0 = split * a.split;
  if (k0 >= n_keys) return;
  const int k1 = min(k0 + a.split, n_keys);
  const int n_splits = (n_keys + a.split - 1) / a.split;
  const int g = z / (a.group / GT);
  const int h0 = g * a.group + (z % (a.group / GT)) * GT;

  // query heads of this workgroup, pre-scaled into log2 units
  float qf[GT][EPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const int64_t qoff = ((int64_t)t * a.num_q_heads + h0 + hh) * D + cl * EPL;
    const uint4 qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) + qoff * IO::kEsz);
    IO::widen(qv, qf[hh]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[hh][e] *= a.scale_log2;
  }

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  const int64_t rs = (int64_t)a.num_kv_heads * D;          // elements per token row
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + ((int64_t)g * D + cl * EPL) * IO::kEsz;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + ((int64_t)g * D + cl * EPL) * IO::kEsz;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
  const int kb0 = k0 / kBlock;
  const int kb1 = (k1 + kBlock - 1) / kBlock;

  auto load_block = [&](int blk, uint4* kr, uint4* vr) {
    const int64_t phys = table[blk];
    const int64_t base = phys * kBlock * rs;
#pragma unroll
    for (int r = 0; r < LPB; ++r) {
      const int64_t off = (base + (int64_t)(r * RPL + rg) * rs) * IO::kEsz;
      kr[r] = *reinterpret_cast<const uint4*>(kbase + off);
      vr[r] = *reinterpret_cast<const uint4*>(vbase + off);
    }
  };

  auto consume_block = [&](int blk, const uint4* kr, const uint4* vr) {
    float sc[LPB][GT];
#pragma unroll
    for (int r = 0; r < LPB; ++r) {
      float kf[EPL];
      IO::widen(kr[r], kf);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[hh][e], kf[e], d);
        sc[r][hh] = group_sum<LPR>(d);
      }
    }
    const int key0 = blk * kBlock + rg;
    const bool full = (blk + 1) * kBlock <= k1;
    float vf[LPB][EPL];
#pragma unroll
    for (int r = 0; r < LPB; ++r) {
      IO::widen(vr[r], vf[r]);
      if (!full && key0 + r * RPL >= k1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[r][e] = 0.f;      // slots past the last visible key
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) sc[r][hh] = -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float bm = sc[0][hh];
#pragma unroll
      for (int r = 1; r < LPB; ++r) bm = fmaxf(bm, sc[r][hh]);
      const float mn = fmaxf(m[hh], bm);
      if (mn == -INFINITY) continue;                       // nothing visible yet in this group
      const float alpha = fast_exp2(m[hh] - mn);           // 0 when m was -inf
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int r = 0; r < LPB; ++r) {
        const float p = fast_exp2(sc[r][hh] - mn);
        ps += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(p, vf[r][e], acc[hh][e]);
      }
      l[hh] = l[hh] * alpha + ps;
      m[hh] = mn;
    }
  };

  for (int blk = kb0 + w; blk < kb1; blk += 8) {
    uint4 ka[LPB], va[LPB], kb_[LPB], vb_[LPB];
    const bool two = blk + 4 < kb1;
    load_block(blk, ka, va);
    if (two) load_block(blk + 4, kb_, vb_);
    consume_block(blk, ka, va);
    if (two) consume_block(blk + 4, kb_, vb_);
  }

  // merge the row groups of this wave (lanes with equal `cl` hold the same elements)
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const float mw = wave_max_over_groups(m[hh], LPR);
    const float f = (m[hh] == -INFINITY) ? 0.f : fast_exp2(m[hh] - mw);
    const float lw = wave_sum_over_groups(l[hh] * f, LPR);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = wave_sum_over_groups(acc[hh][e] * f, LPR);
    if (lane == 0) {
      sm_m[w][hh] = mw;
      sm_l[w][hh] = lw;
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[w][hh][cl * EPL + e] = acc[hh][e];
    }
  }
  __syncthreads();

  // merge the four waves and write either the final row or this split's partial
  for (int idx = threadIdx.x; idx < GT * D; idx += blockDim.x) {
    const int hh = idx / D;
    const int dd = idx % D;
    float mm = sm_m[0][hh];
#pragma unroll
    for (int i = 1; i < 4; ++i) mm = fmaxf(mm, sm_m[i][hh]);
    float ll = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = (sm_m[i][hh] == -INFINITY) ? 0.f : fast_exp2(sm_m[i][hh] - mm);
      ll += sm_l[i][hh] * f;
      o += sm_o[i][hh][dd] * f;
    }
    const int h = h0 + hh;
    if (n_splits == 1) {
      IO::store(a.out, ((int64_t)t * a.num_q_heads + h) * D + dd, o / ll);
    } else {
      const int64_t pidx = ((int64_t)row * a.max_splits + split) * a.num_q_heads + h;
      a.part_o[pidx * D + dd] = o;
      if (dd == 0) {
        a.part_ml[pidx * 2] = mm;
        a.part_ml[pidx * 2 + 1] = ll;
      }
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  using IO = Io<BF16>;
  const int row = blockIdx.x / a.num_q_heads;
  const int h = blockIdx.x % a.num_q_heads;
  int b, t, n_keys;
  if (!resolve_row(a, row, b, t, n_keys)) return;
  const int n_splits = (n_keys + a.split - 1) / a.split;
  if (n_splits <= 1) return;                                // written directly by the split kernel
  const int64_t pbase = (int64_t)row * a.max_splits * a.num_q_heads + h;
  float mm = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mm = fmaxf(mm, a.part_ml[(pbase + (int64_t)s * a.num_q_heads) * 2]);
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  float ll = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t p = pbase + (int64_t)s * a.num_q_heads;
    const float f = fast_exp2(a.part_ml[p * 2] - mm);
    ll += a.part_ml[p * 2 + 1] * f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[i] = fmaf(a.part_o[p * D + threadIdx.x + 64 * i], f, o[i]);
  }
  const float inv = 1.f / ll;
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    IO::store(a.out, ((int64_t)t * a.num_q_heads + h) * D + threadIdx.x + 64 * i, o[i] * inv);
}

namespace {
template <int D, bool BF16>
hipError_t split_dispatch(const DecodeArgs& a, hipStream_t s) {
  const int64_t nz = (int64_t)a.num_kv_heads * (a.group / a.heads_per_wg);
  const int64_t grid = nz * a.max_splits * a.num_rows;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(256);
  switch (a.heads_per_wg) {
    case 1: decode_split_kernel<D, 1, BF16><<<g, blk, 0, s>>>(a); break;
    case 2: decode_split_kernel<D, 2, BF16><<<g, blk, 0, s>>>(a); break;
    case 4: decode_split_kernel<D, 4, BF16><<<g, blk, 0, s>>>(a); break;
    case 8: decode_split_kernel<D, 8, BF16><<<g, blk, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s) {
  if (head_dim == 128) return bf16 ? split_dispatch<128, true>(a, s) : split_dispatch<128, false>(a, s);
  if (head_dim == 64) return bf16 ? split_dispatch<64, true>(a, s) : split_dispatch<64, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s) {
  const int64_t grid = (int64_t)a.num_rows * a.num_q_heads;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(64);
  if (head_dim == 128) {
    if (bf16) decode_merge_kernel<128, true><<<g, blk, 0, s>>>(a);
    else decode_merge_kernel<128, false><<<g, blk, 0, s>>>(a);
  } else if (head_dim == 64) {
    if (bf16) decode_merge_kernel<64, true><<<g, blk, 0, s>>>(a);
    else decode_merge_kernel<64, false><<<g, blk, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
