// pa_prefill.hip -- causal attention tiles for requests with q_len >= 2 (one-shot prefill and
// chunked prefill), on bf16 MFMA, plus the device-side tile planner.
//
// A prefill row block attends over every key up to its own position (P3 §2.1) and a chunk
// additionally reads the keys of all earlier chunks from the cache (P4 "块大小怎样取舍": chunk 15
// reads the KV of the 14 chunks before it).  The S x S score matrix is never stored: K/V tiles are
// staged in LDS and consumed with an online softmax (P3 §2.1, P1 §2.1 describe the on-chip tiling
// idea; the tiling here is CDNA4's own).  Arithmetic intensity is ~S FLOP/byte, so this part is a
// dense contraction and runs on the matrix cores.
//
// Tile shape: 128 query rows x 64 keys per step, four waves of 32 rows.  A query row is a
// (position, query head) pair; the Hq/Hkv heads of one KV group are packed into the rows of the
// same tile so that each K/V tile is loaded once for the whole group.  Per wave and key tile:
//   S^T (64 keys x 32 rows) = K (64 x d) . Q^T (d x 32)     -- v_mfma_f32_32x32x16_bf16
//   online softmax on S^T in registers (lane = query row, 16 keys per lane and sub-tile)
//   O^T (d x 32 rows)     += V^T (d x 64) . P^T (64 x 32)   -- P^T stays in registers
// V is written to LDS transposed, with keys permuted inside each 16-key step so that the eight
// keys a lane needs for one MFMA operand are contiguous.  Key tiles entirely above the causal
// diagonal of the last row are never visited; only tiles crossing the diagonal are masked.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

namespace {

// LDS column of key kappa (0..15) inside a 16-key MFMA k-step: the accumulator layout of S^T
// gives lane half a the keys {4a..4a+3, 8+4a..8+4a+3}; they are stored as slots 8a..8a+7.
__device__ __forceinline__ int vt_slot(int kappa) {
  return 8 * ((kappa >> 2) & 1) + 4 * (kappa >> 3) + (kappa & 3);
}

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_tile_kernel(TileArgs a) {
  constexpr int KS = D + 8;                 // K tile row stride (elements)
  constexpr int VT = kTileKeys + 8;         // V^T tile row stride (elements)
  constexpr int NKK = D / 16;               // MFMA k-steps over d
  constexpr int NDT = D / 32;               // 32-wide d tiles of O^T
  constexpr int CPR = D / 8;                // 16-byte pieces per K/V row
  constexpr int PAIRS = (kTileKeys / 2) * CPR;
  static_assert(PAIRS % 256 == 0, "staging split");
  __shared__ __align__(16) uint16_t Ks[kTileKeys * KS];
  __shared__ __align__(16) uint16_t Vt[D * VT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // workgroup -> (tile slot, KV head); WG i runs on XCD i % 8, so the KV heads are dealt out to
  // the XCDs and all tiles of a head share one L2.
  int slot, g;
  {
    const int i = blockIdx.x;
    if ((a.num_kv_heads & 7) == 0) {
      const int hpx = a.num_kv_heads >> 3;
      const int x = i & 7, k = i >> 3;
      g = x * hpx + (k % hpx);
      slot = k / hpx;
    } else {
      g = i % a.num_kv_heads;
      slot = i / a.num_kv_heads;
    }
  }
  if (slot >= *a.num_tiles) return;
  const int4 tile = a.tiles[slot];
  const int b = tile.x, q_off = tile.y, n_pos = tile.z;
  const int q0 = a.qsl[b];
  const int ql = a.qsl[b + 1] - q0;
  const int sl = a.seq_lens[b];
  const int ctx = sl - ql;
  const int G = a.group;

  const int rho = 32 * w + l32;                  // this lane's query row within the tile
  const int pl = rho / G;
  const int hh = rho - pl * G;
  const bool row_ok = (pl < a.pos_per_tile) && (pl < n_pos);
  const int pos = ctx + q_off + pl;              // absolute position of the row
  const int64_t t = (int64_t)q0 + q_off + pl;
  const int h = g * G + hh;

  bf16x8 qreg[NKK];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + (((t * a.num_q_heads + h) * D) + 8 * half) * 2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (row_ok) {
        qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 32);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[kk][e] = (__bf16)0.f;
      }
    }
  }

  const int kv_end = min(sl, ctx + q_off + n_pos);   // keys needed by the last row of the tile
  const int n_kt = (kv_end + kTileKeys - 1) / kTileKeys;
  const int first_pos = ctx + q_off;
  const float c = a.scale_log2;
  const int64_t rs = (int64_t)a.num_kv_heads * D;    // elements per cache token row
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * D * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * D * 2;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  float m_run = -INFINITY, l_run = 0.f;
  floatx16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[dt][v] = 0.f;

  for (int kt = 0; kt < n_kt; ++kt) {
    // ---- stage K (row-major) and V (transposed, permuted) for keys kt*64 .. kt*64+63 ----
#pragma unroll
    for (int it = 0; it < PAIRS / 256; ++it) {
      const int pc = tid + 256 * it;
      const int kp = pc / CPR;
      const int dc = pc - kp * CPR;
      const int j0 = kt * kTileKeys + 2 * kp;
      uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
      if (j0 < sl) {
        const int64_t phys = table[j0 >> 4];
        const int64_t off = ((phys * kBlock + (j0 & 15)) * rs + dc * 8) * 2;
        k0 = *reinterpret_cast<const uint4*>(kbase + off);
        v0 = *reinterpret_cast<const uint4*>(vbase + off);
        if (j0 + 1 < sl) {
          k1 = *reinterpret_cast<const uint4*>(kbase + off + rs * 2);
          v1 = *reinterpret_cast<const uint4*>(vbase + off + rs * 2);
        }
      }
      *reinterpret_cast<uint4*>(&Ks[(2 * kp) * KS + dc * 8]) = k0;
      *reinterpret_cast<uint4*>(&Ks[(2 * kp + 1) * KS + dc * 8]) = k1;
      const int key = 2 * kp;
      const int col = (key & ~15) + vt_slot(key & 15);
      uint32_t* vt32 = reinterpret_cast<uint32_t*>(Vt);
      const int r0 = dc * 8;
      vt32[((r0 + 0) * VT + col) >> 1] = pair_lo(v0.x, v1.x);
      vt32[((r0 + 1) * VT + col) >> 1] = pair_hi(v0.x, v1.x);
      vt32[((r0 + 2) * VT + col) >> 1] = pair_lo(v0.y, v1.y);
      vt32[((r0 + 3) * VT + col) >> 1] = pair_hi(v0.y, v1.y);
      vt32[((r0 + 4) * VT + col) >> 1] = pair_lo(v0.z, v1.z);
      vt32[((r0 + 5) * VT + col) >> 1] = pair_hi(v0.z, v1.z);
      vt32[((r0 + 6) * VT + col) >> 1] = pair_lo(v0.w, v1.w);
      vt32[((r0 + 7) * VT + col) >> 1] = pair_hi(v0.w, v1.w);
    }
    __syncthreads();

    // ---- S^T = K Q^T : two 32-key sub-tiles ----
    floatx16 S[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[st][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&Ks[(32 * st + l32) * KS + kk * 16 + 8 * half]);
        S[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kk], S[st], 0, 0, 0);
      }
    }

    // ---- causal mask (only on tiles that cross the diagonal of the first row) ----
    if (kt * kTileKeys + kTileKeys - 1 > first_pos) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt * kTileKeys + 32 * st + 8 * (v >> 2) + 4 * half + (v & 3);
          if (key > pos) S[st][v] = -INFINITY;
        }
    }

    // ---- online softmax (scores in log2 units via c = scale * log2 e) ----
    float tm = S[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) tm = fmaxf(tm, S[st][v]);
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m_run, tm);
    const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - mn) * c);
    const float mc = mn * c;
    bf16x8 P[4];
    float ps = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(S[st][v], c, -mc));
        ps += p;
        P[2 * st + (v >> 3)][v & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + ps;
    m_run = mn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[dt][v] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(&Vt[(32 * dt + l32) * VT + 16 * kk + 8 * half]);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, P[kk], O[dt], 0, 0, 0);
      }
    __syncthreads();
  }

  // ---- epilogue: O / l, round to bf16, store (lane holds 4 consecutive d per group) ----
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / lt;
  if (row_ok) {
    char* op = reinterpret_cast<char*>(a.out) + ((t * a.num_q_heads + h) * D) * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int dd = 32 * dt + 8 * grp + 4 * half;
        uint2 pk;
        pk.x = pack_bf16x2(O[dt][4 * grp + 0] * inv, O[dt][4 * grp + 1] * inv);
        pk.y = pack_bf16x2(O[dt][4 * grp + 2] * inv, O[dt][4 * grp + 3] * inv);
        *reinterpret_cast<uint2*>(op + dd * 2) = pk;
      }
  }
}

// One workgroup: per request, ceil(q_len / pos_per_tile) tiles for every request with q_len >= 2,
// written with the last (longest) row block of each request first.
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* qsl, int num_seqs, int pos_per_tile,
                                                         int4* tiles, int* num_tiles) {
  __shared__ int scan[256];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < num_seqs; c0 += 256) {
    const int b = c0 + tid;
    int ql = 0, cnt = 0;
    if (b < num_seqs) {
      ql = qsl[b + 1] - qsl[b];
      cnt = ql >= 2 ? (ql + pos_per_tile - 1) / pos_per_tile : 0;
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int excl = base + scan[tid] - cnt;
    for (int i = 0; i < cnt; ++i) {
      const int qi = cnt - 1 - i;
      tiles[excl + i] = make_int4(b, qi * pos_per_tile, min(pos_per_tile, ql - qi * pos_per_tile), 0);
    }
    __syncthreads();
    if (tid == 255) base += scan[255];
    __syncthreads();
  }
  if (tid == 0) *num_tiles = base;
}

hipError_t launch_plan_tiles(const int32_t* qsl, int num_seqs, int pos_per_tile, int4* tiles, int* num_tiles,
                             hipStream_t s) {
  plan_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(qsl, num_seqs, pos_per_tile, tiles, num_tiles);
  return hipGetLastError();
}

hipError_t launch_prefill_tile(const TileArgs& a, int head_dim, hipStream_t s) {
  const int64_t grid = (int64_t)a.num_slots * a.num_kv_heads;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (head_dim == 128) prefill_tile_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  else if (head_dim == 64) prefill_tile_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
