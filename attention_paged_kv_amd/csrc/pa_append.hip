// pa_append.hip -- KV append into the paged cache, and the check-mode index validator.
//
// Append: each new token's K and V rows (Hkv*d elements each) are copied bit for bit to the
// cache slot given for it (P3 §2.3: only K and V are cached; P1 §2.2: written at the page
// index).  With the position-major cache layout a token's row is contiguous in the cache, so
// the scatter is a coalesced 16-byte-per-lane copy: consecutive lanes move consecutive 16-byte
// pieces of the same row.
//
// 8-bit caches (P2 §4.3, §5.4: INT8 KV with per-channel calibration): the append quantises
// instead of copying.  Element c of a token row (c = head * d + channel) becomes
// clamp(rne(x / s_c), -127, 127) with the division rounded to fp32 and NaN mapped to 0.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t per_row = a.row_bytes >> 4;                 // 16-byte pieces per token row
  const int64_t total = a.num_tokens * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const int64_t tok = c / per_row;
    const int64_t piece = c - tok * per_row;
    const int32_t slot = a.slot_mapping[tok];
    if (slot < 0) continue;                                  // padding token
    const int64_t src = tok * per_row + piece;
    const int64_t dst = (int64_t)slot * per_row + piece;
    const uint4 kv = reinterpret_cast<const uint4*>(a.k)[src];
    const uint4 vv = reinterpret_cast<const uint4*>(a.v)[src];
    reinterpret_cast<uint4*>(a.k_cache)[dst] = kv;
    reinterpret_cast<uint4*>(a.v_cache)[dst] = vv;
  }
}

__device__ __forceinline__ uint32_t quantize(float x, float s) {
  float r = __fdiv_rn(x, s);
  if (r != r) return 0u;
  r = fminf(fmaxf(rintf(r), -127.f), 127.f);
  return (uint32_t)(int)r & 0xFFu;
}

__device__ __forceinline__ uint2 quantize8(const uint4& x, const float4& s0, const float4& s1) {
  uint2 o;
  o.x = quantize(bf16_lo(x.x), s0.x) | quantize(bf16_hi(x.x), s0.y) << 8 | quantize(bf16_lo(x.y), s0.z) << 16 |
        quantize(bf16_hi(x.y), s0.w) << 24;
  o.y = quantize(bf16_lo(x.z), s1.x) | quantize(bf16_hi(x.z), s1.y) << 8 | quantize(bf16_lo(x.w), s1.z) << 16 |
        quantize(bf16_hi(x.w), s1.w) << 24;
  return o;
}

// One lane: 16 elements (two 16-byte loads per tensor in, one 16-byte store of codes out).  All
// loads are taken into registers before either store, so the stores cannot serialise them.
__global__ __launch_bounds__(256) void append_i8_kernel(AppendArgs a) {
  const int64_t per_row = a.row_bytes >> 5;                 // 16-element pieces per token row
  const int64_t total = a.num_tokens * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const int64_t tok = c / per_row;
    const int64_t piece = c - tok * per_row;
    const int32_t slot = a.slot_mapping[tok];
    if (slot < 0) continue;
    const uint4* kin = reinterpret_cast<const uint4*>(a.k) + 2 * c;
    const uint4* vin = reinterpret_cast<const uint4*>(a.v) + 2 * c;
    const float4* ksp = reinterpret_cast<const float4*>(a.k_scale) + 4 * piece;
    const float4* vsp = reinterpret_cast<const float4*>(a.v_scale) + 4 * piece;
    const uint4 k0 = kin[0], k1 = kin[1], v0 = vin[0], v1 = vin[1];
    const float4 ks0 = ksp[0], ks1 = ksp[1], ks2 = ksp[2], ks3 = ksp[3];
    const float4 vs0 = vsp[0], vs1 = vsp[1], vs2 = vsp[2], vs3 = vsp[3];
    const uint2 ka = quantize8(k0, ks0, ks1), kb = quantize8(k1, ks2, ks3);
    const uint2 va = quantize8(v0, vs0, vs1), vb = quantize8(v1, vs2, vs3);
    const int64_t dst = (int64_t)slot * per_row + piece;
    reinterpret_cast<uint4*>(a.k_cache)[dst] = make_uint4(ka.x, ka.y, kb.x, kb.y);
    reinterpret_cast<uint4*>(a.v_cache)[dst] = make_uint4(va.x, va.y, vb.x, vb.y);
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t total = a.num_tokens * (a.row_bytes >> (a.k_scale ? 5 : 4));
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (a.k_scale) append_i8_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  else append_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Check mode: validates the index arguments on the device before any data kernel runs.
// result[0] = 1 once an error is recorded; result[1] = code; result[2] = index; result[3] = value.
// ------------------------------------------------------------------------------------------
__device__ void report(int* r, int code, int index, int value) {
  if (atomicCAS(&r[0], 0, 1) == 0) {
    r[1] = code;
    r[2] = index;
    r[3] = value;
  }
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a, unsigned* bitmap) {
  const int tid = threadIdx.x + blockIdx.x * blockDim.x;
  const int nthr = blockDim.x * gridDim.x;
  if (a.slot_mapping) {
    for (int i = tid; i < a.num_tokens; i += nthr) {
      const int s = a.slot_mapping[i];
      if (s < 0) continue;
      if ((int64_t)s >= a.num_slots) { report(a.result, 1, i, s); continue; }
      const unsigned bit = 1u << (s & 31);
      const unsigned old = atomicOr(&bitmap[s >> 5], bit);
      if (old & bit) report(a.result, 2, i, s);
    }
  }
  if (a.block_tables) {
    if (tid == 0) {
      if (a.qsl[0] != 0) report(a.result, 3, 0, a.qsl[0]);
      if (a.qsl[a.num_seqs] != a.num_q_tokens) report(a.result, 4, a.num_seqs, a.qsl[a.num_seqs]);
    }
    for (int b = tid; b < a.num_seqs; b += nthr) {
      const int ql = a.qsl[b + 1] - a.qsl[b];
      const int sl = a.seq_lens[b];
      if (ql < 1) { report(a.result, 5, b, ql); continue; }
      if (a.max_q_len > 0 && ql > a.max_q_len) { report(a.result, 9, b, ql); continue; }
      if (sl < ql) { report(a.result, 6, b, sl); continue; }
      if (sl > a.max_blocks * kBlock) { report(a.result, 7, b, sl); continue; }
      const int nb = (sl + kBlock - 1) / kBlock;
      const int j0 = max(0, sl - ql - a.window + 1) / kBlock;   // older blocks are never read
      for (int j = j0; j < nb; ++j) {
        const int blk = a.block_tables[(int64_t)b * a.max_blocks + j];
        if (blk < 0 || blk >= a.num_blocks) { report(a.result, 8, b * a.max_blocks + j, blk); break; }
      }
    }
  }
}

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
  unsigned* bitmap = nullptr;
  if (a.slot_mapping) {
    const size_t words = (size_t)((a.num_slots + 31) / 32);
    hipError_t e = hipMalloc(&bitmap, words * sizeof(unsigned));
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(bitmap, 0, words * sizeof(unsigned), s);
    if (e != hipSuccess) { (void)hipFree(bitmap); return e; }
  }
  check_kernel<<<dim3(64), dim3(256), 0, s>>>(a, bitmap);
  hipError_t e = hipGetLastError();
  if (bitmap) {
    hipError_t e2 = hipStreamSynchronize(s);
    const hipError_t e3 = hipFree(bitmap);
    if (e == hipSuccess) e = e2;
    if (e == hipSuccess) e = e3;
  }
  return e;
}

}  // namespace pa
