// pa_decode_i8.hip -- split-KV attention for decode rows (and rows of a few tokens to verify) over
// an 8-bit cache.
//
// The cache holds int8 codes with one fp32 scale per (KV head, channel) for K and for V (P2 §4.3
// and §5.4: INT8 halves the bytes a decode step must read; calibration is per channel).  The pass
// stays bound by HBM bandwidth (P3 §3.2), now over half the bytes.  Work split, head-quad
// workgroups, online softmax in log2 units and the partial layout are those of the bf16 decode
// kernel; what changes is how the codes meet the matrix cores (fp16 products, fp32 accumulation):
//   * Codes become fp16 with byte permutes: u = code + 128 (an XOR of the sign bit) placed under the
//     fp16 exponent of 1024 is exactly 1024 + u = 1152 + code.
//   * K: the channel scale is folded into the query, q'[c] = q[c] * k_scale[g][c], scaled by a power
//     of two per head so that max |q'| lies in [0.5, 1) and rounded once to fp16 (the B operand).
//     K enters as 1152 + code, so every score of a head carries the same bias 1152 * sum_c q'[c];
//     it is subtracted once per 32 keys, before the softmax.
//   * V: the channel scale factors out of the sum over keys, so O is multiplied by v_scale[g][c]
//     once at the end.  V codes are staged in LDS by direct global->LDS loads and read back with
//     the 8-bit transpose read (ds_read_b64_tr_b8), which hands each lane 8 keys of one channel
//     (the A operand of a 16x16x32 product); one packed fp16 subtraction of 1152 recovers the
//     exact codes.
// Keys are consumed in units of 32 (two cache blocks): S^T of both blocks, one softmax update,
// then O^T += V^T (d x 32 keys) . P^T (32 keys x heads) with v_mfma_f32_16x16x32_f16.  O is only
// rescaled when a head's running max grows by more than 2^8, so P <= 2^8 fits fp16.  Masked keys
// need no zeroing of V: every code is a finite number under a zero probability.
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_rows.h"

namespace pa {

namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kCodeBias = 1152.f;          // value of fp16 bits 0x6400 | (code ^ 0x80)

// Per-wave staging (a wave's own head, D bytes per staged row): the physical 16-byte chunk of
// logical chunk q in row r of staged V block blk is q ^ vswz(blk, r), so that the transpose reads of
// a wave hit every LDS bank once, and in staged K row r it is q ^ kswz(r), so that the 16 rows read
// by one 16-lane group for the same logical chunk land on distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int blk, int r) {
  if constexpr (D == 128) return ((r ^ (r >> 2)) & 3) | (blk << 2);
  else return (((r >> 1) ^ (r >> 2)) & 1) | (blk << 1);
}
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// Whole-row staging (the workgroup's NW heads, NW * D bytes per staged row, a multiple of 256, so
// every row starts on the same LDS bank): physical chunk p of staged row r holds logical chunk
// p ^ row_swz(r) of the NW heads' bytes, for K and V alike; the 16 rows that a 16-lane group reads
// for one logical chunk land on 16 different bank groups, and so do the rows of a transpose read.
__device__ __forceinline__ int row_swz(int r) { return r & 15; }

// Eight int8 codes (little-endian in lo, hi) as fp16 values 1152 + code, exactly.  v_perm_b32
// picks bytes of {0x64646464 : x}: selector 0-3 = byte of x, 4 = 0x64.
__device__ __forceinline__ f16x8 codes_biased_f16(uint32_t lo, uint32_t hi) {
  lo ^= 0x80808080u;
  hi ^= 0x80808080u;
  uint4 r;
  r.x = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}

// Eight int8 codes as exact fp16 codes.
__device__ __forceinline__ f16x8 codes_f16(uint32_t lo, uint32_t hi) {
  const f16x8 b = codes_biased_f16(lo, hi);
  const f16x2 nb = f16x2{(_Float16)-kCodeBias, (_Float16)-kCodeBias};
  f16x8 r;
  const f16x2 r0 = f16x2{b[0], b[1]} + nb, r1 = f16x2{b[2], b[3]} + nb;
  const f16x2 r2 = f16x2{b[4], b[5]} + nb, r3 = f16x2{b[6], b[7]} + nb;
  r[0] = r0[0]; r[1] = r0[1]; r[2] = r1[0]; r[3] = r1[1];
  r[4] = r2[0]; r[5] = r2[1]; r[6] = r3[0]; r[7] = r3[1];
  return r;
}

// 8-bit transpose read: in each 16-lane group, lane 2e + h gives the address of bytes 8h..8h+7 of
// row e of an 8 x 16-byte tile; lane j receives column j of the tile (rows 0..7).
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(const __attribute__((address_space(3))) char*)p);
}

}  // namespace

// NW = 4 waves per workgroup, one adjacent KV head each.  K and V codes of a 32-key unit are copied
// by direct global->LDS loads (inline assembly waited for with explicit vmcnt counts, see dma16)
// into one slot of a double buffer while the other slot is computed, in one of two forms:
//   * per wave (ROWS = false): each wave copies its own head's D-byte pieces of the unit's 32 token
//     rows into a buffer of its own; the waves run independently, with no barriers, and the wait
//     leaves the next unit's copies in flight during the arithmetic;
//   * whole rows (ROWS = true): the workgroup stages the NW heads' NW * D contiguous bytes of each
//     token row, the 32 rows split among the waves, each 1 KiB copy covering 1024 / (NW * D) rows;
//     a barrier per unit ends unit u's copies (and every wave's reads of unit u - 1), after which
//     the copies of unit u + 1 go out and stay in flight while unit u is computed.
// Whole rows turn each copy into runs of 256 or 512 contiguous bytes instead of one head's 64 or
// 128; that pays where cache rows are 4 KiB or wider and costs where they are narrower (the launch
// picks the form by the row width).
template <int D, int NW, bool ROWS, bool STREAM>
__global__ __launch_bounds__(64 * NW, 2) void decode_i8_kernel(DecodeArgs a) {
  static_assert(NW == 4, "whole-row staging splits the unit's 32 rows 8 per wave");
  constexpr int NKK = D / 32;                 // 16x16x32 k-steps over d for S^T (8 codes per lane)
  constexpr int NT = D / 16;                  // 16-row d tiles of O^T
  constexpr int KL = D / 64;                  // 16-byte K loads per lane and block
  constexpr int CPH = D / 16;                 // 16-byte chunks per head in a row
  constexpr int RB = ROWS ? NW * D : D;       // bytes of one staged token row
  constexpr int CPS = RB / 16;                // 16-byte chunks per staged row
  constexpr int RPC = 1024 / RB;              // rows per wave-wide 1 KiB copy
  constexpr int RPW = ROWS ? 2 * kBlock / NW : 2 * kBlock;   // rows of a unit copied by each wave
  constexpr int CPW = RPW / RPC;              // copies per wave, unit and tensor
  constexpr int UB = 2 * kBlock * RB;         // bytes of one staged 32-key unit (two blocks)
  constexpr int NCP = 2 * CPW;                // copies per wave and unit (K and V)
  static_assert(!ROWS || (RB % 256 == 0 && CPS <= 64 && RPW % RPC == 0 && RPW <= kBlock), "staging shape");
  // [slot][K unit, V unit], per wave in the per-wave form
  __shared__ __align__(16) char sKV[2 * (ROWS ? 1 : NW) * 2 * UB];

  // unit: (row, split) -- or, in stream mode, run pw of the rows' concatenated blocks, taken as
  // one pass per row it meets -- for one head group and column group (fastest); the wave's KV head
  // is NW * group + w.  Columns
  // are the row's (position, query head) pairs of that KV head, heads_per_wg of them per group: a
  // decode row has one position, a row of tokens to verify q_len <= qmax of them, each column
  // masked to its own causal (and window) range.
  const int nzh = (a.qmax * a.group + a.heads_per_wg - 1) / a.heads_per_wg;
  const int nq = (a.num_kv_heads + NW - 1) / NW;
  const int nz = nq * nzh;
  const int z = blockIdx.x % nz;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g0 = NW * (z / nzh);                           // the workgroup's first KV head
  const int g = g0 + w;
  const bool live = g < a.num_kv_heads;
  if (!ROWS && !live) return;                              // (whole rows: such a wave only copies)
  const int c0 = (z % nzh) * a.heads_per_wg;               // first column of this group

  const int lane = threadIdx.x & (kWave - 1);
  const int col = lane & 15;                  // S^T / O^T column; also the K row loaded
  const int grp = lane >> 4;

  const int64_t rs = (int64_t)a.num_kv_heads * D;          // bytes per cache token row
  const int64_t blkbytes = kBlock * rs;
  // K operand j of a block: key row `col`, this head's logical chunk grp + 4j (channels 64j + 16grp
  // .. +16); the second block's rows are kBlock rows on, with the same swizzle
  uint32_t k_rd[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j)
    k_rd[j] = ROWS ? col * RB + (((w * CPH + grp + 4 * j) ^ row_swz(col)) * 16)
                   : col * RB + (((grp + 4 * j) ^ kswz<D>(col)) * 16);
  // copy i of this wave: lane -> staged row ur = (ROWS ? RPW*w : 0) + RPC*i + lane / CPS of the unit
  // (row ur % 16 of its block ur / 16), physical chunk lane % CPS, which holds the swizzled logical
  // chunk of the staged bytes; offsets from the block's first byte.  Whole rows: a chunk of a head
  // past the last one (the last group of a cache whose head count is no multiple of NW) loads the
  // first head's chunk instead, which stays in bounds and is never read, and K and V share the layout.
  const int nh = min(NW, a.num_kv_heads - g0);
  uint32_t k_lane[CPW], v_lane[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int ur = (ROWS ? RPW * w : 0) + RPC * i + lane / CPS;
    const int sb = ur / kBlock, r = ur % kBlock;
    if constexpr (ROWS) {
      int q = (lane % CPS) ^ row_swz(ur);
      if (q >= nh * CPH) q %= CPH;
      k_lane[i] = v_lane[i] = (uint32_t)(r * rs) + (uint32_t)(g0 * D + q * 16);
    } else {
      k_lane[i] = (uint32_t)(r * rs) + (uint32_t)(g * D + (((lane % CPS) ^ kswz<D>(r)) * 16));
      v_lane[i] = (uint32_t)(r * rs) + (uint32_t)(g * D + (((lane % CPS) ^ vswz<D>(sb, r)) * 16));
    }
  }
  // transpose read of tile tt: lane 2e + hh of group grp -> key e of the group, i.e. staged block
  // e / 4, row 4grp + e % 4, this head's channels 16tt + 8hh .. +7
  uint32_t tr_off[NT];
  {
    const int e = col >> 1, hh = col & 1;
    const int sb = e >> 2, rr = 4 * grp + (e & 3), r = kBlock * sb + rr;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      tr_off[tt] = ROWS ? r * RB + (((w * CPH + tt) ^ row_swz(r)) * 16) + 8 * hh
                        : r * RB + ((tt ^ vswz<D>(sb, rr)) * 16) + 8 * hh;
  }

  // unit u = blocks 2u and 2u + 1 of a pass; a missing second block is replaced by the first
  // (valid memory) and all its keys are masked.  The slot of unit u is wave_buf + (u & 1) * SLOT.
  constexpr int SLOT = (ROWS ? 1 : NW) * 2 * UB;
  char* const wave_buf = ROWS ? sKV : sKV + w * 2 * UB;

  // One pass over keys [k0, k1) of a row: its partial is number `split` of the row's n_splits (the
  // output itself when n_splits is 1).  Every return before the key loop is per workgroup.
  auto pass = [&](int row, int b, int t, int n_keys, int ql, int k0, int k1, int split, int n_splits) {
    const int ctx = n_keys - ql;                             // keys before the row's first position
    const int lo_max = first_visible(a, n_keys);             // oldest key the last position sees
    const int ncol_all = ql * a.group;
    if (c0 >= ncol_all) return;                              // no column of this group in the row

    const bool on = col < a.heads_per_wg && c0 + col < ncol_all;
    const int cr = on ? (c0 + col) / a.group : 0;            // the column's position in the row
    const int h = g * a.group + (on ? (c0 + col) % a.group : 0);
    const int nvis = ctx + cr + 1;                           // keys [lo_c, nvis) are the column's
    const int lo_c = first_visible(a, nvis);

    // q' = q * k_scale * 2^-e as the B operand.  Step kk covers channels 64(kk/2) + 16grp + 8(kk%2)
    // + [0, 8) (any order of the channels works as long as K uses the same one).  The four lanes
    // of a column (grp = 0..3) share e, the scaled softmax factor c and the score bias.
    // (Loaded by load_q after the first unit's copies are issued, so the two latencies overlap.)
    f16x8 qb[NKK];
    float c, bias;
    auto load_q = [&]() {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)(t + cr) * a.num_q_heads + h) * D;
      const float* ksp = a.k_scale + (int64_t)g * D;
      float qf[NKK][8];
      float mx = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int d0 = 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1);
        const uint4 v = on ? *reinterpret_cast<const uint4*>(qp + d0) : make_uint4(0, 0, 0, 0);
        const float4 s0 = *reinterpret_cast<const float4*>(ksp + d0);
        const float4 s1 = *reinterpret_cast<const float4*>(ksp + d0 + 4);
        qf[kk][0] = bf16_lo(v.x) * s0.x;
        qf[kk][1] = bf16_hi(v.x) * s0.y;
        qf[kk][2] = bf16_lo(v.y) * s0.z;
        qf[kk][3] = bf16_hi(v.y) * s0.w;
        qf[kk][4] = bf16_lo(v.z) * s1.x;
        qf[kk][5] = bf16_hi(v.z) * s1.y;
        qf[kk][6] = bf16_lo(v.w) * s1.z;
        qf[kk][7] = bf16_hi(v.w) * s1.w;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(qf[kk][i]));
      }
      mx = xor16_max(mx);
      mx = xor32_max(mx);
      int e = 0;
      if (mx > 0.f) frexpf(mx, &e);                           // mx = f * 2^e, f in [0.5, 1)
      float qs = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const _Float16 h = (_Float16)ldexpf(qf[kk][i], -e);
          qb[kk][i] = h;
          qs += (float)h;
        }
      qs = xor16_sum(qs);
      qs = xor32_sum(qs);
      bias = kCodeBias * qs;                                  // score offset from the biased K codes
      c = ldexpf(a.scale_log2, e);                            // log2-unit factor of this column's scores
    };

    const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
    const int kb0 = k0 / kBlock;
    const int nb = (k1 + kBlock - 1) / kBlock - kb0;         // blocks of this pass
    const int nu = (nb + 1) >> 1;                            // 32-key units
    // lane i: id of the pass's block ids_base + i; a pass of more than 64 blocks (a stream-mode
    // piece) loads the next 64 when its units reach them
    int ids_base = 0;
    int ids = lane < nb ? table[kb0 + lane] : 0;

    float m = -INFINITY, lsum = 0.f;
    floatx4 O[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) O[tt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int u, int slot) {
      if constexpr (!ROWS) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the slot's earlier reads are done
      if (STREAM && 2 * u - ids_base >= kWave) {        // (a split has at most 64 blocks)
        ids_base = 2 * u;
        ids = load_ids_sync(table + kb0 + ids_base, nb - ids_base);
      }
      const int b0 = (ROWS ? min(2 * u + (RPW * w) / kBlock, nb - 1) : 2 * u) - ids_base;
      const int64_t o0 = (int64_t)__builtin_amdgcn_readlane(ids, b0) * blkbytes;
      const int64_t o1 = ROWS ? o0 : (int64_t)__builtin_amdgcn_readlane(ids, min(2 * u + 1, nb - 1) - ids_base) * blkbytes;
      const uint32_t l = __builtin_amdgcn_readfirstlane(lds_u32(wave_buf + slot * SLOT + (ROWS ? RPW * w * RB : 0)));
      const char* kc = reinterpret_cast<const char*>(a.k_cache);
      const char* vc = reinterpret_cast<const char*>(a.v_cache);
#pragma unroll
      for (int i = 0; i < CPW; ++i) dma16(kc + (RPC * i < kBlock ? o0 : o1), k_lane[i], l + 1024 * i);
#pragma unroll
      for (int i = 0; i < CPW; ++i) dma16(vc + (RPC * i < kBlock ? o0 : o1), v_lane[i], l + UB + 1024 * i);
    };

    // one unit; EDGE: it holds keys some column must not see -- past k1 or past a column's position
    // (the pass's last units), or before a column's window (the first units of a row's first pass)
    auto consume = [&](auto edge_tag, int u, int slot) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      const char* kw = wave_buf + slot * SLOT;
      uint4 kr[2 * KL];
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        kr[j] = *reinterpret_cast<const uint4*>(kw + k_rd[j]);
        kr[KL + j] = *reinterpret_cast<const uint4*>(kw + kBlock * RB + k_rd[j]);
      }
      floatx4 sA = floatx4{0.f, 0.f, 0.f, 0.f}, sB = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint4 xa = kr[kk >> 1], xb = kr[KL + (kk >> 1)];
        const f16x8 ka = (kk & 1) ? codes_biased_f16(xa.z, xa.w) : codes_biased_f16(xa.x, xa.y);
        const f16x8 kb = (kk & 1) ? codes_biased_f16(xb.z, xb.w) : codes_biased_f16(xb.x, xb.y);
        sA = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[kk], sA, 0, 0, 0);
        sB = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, qb[kk], sB, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sA[v] -= bias;
        sB[v] -= bias;
      }
      if constexpr (EDGE) {
        const int base = (kb0 + 2 * u) * kBlock;
        const int nhi = min(k1, nvis) - base, nlo = lo_c - base;   // keys [nlo, nhi) of the unit are visible
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ka = 4 * grp + v, kb = kBlock + 4 * grp + v;
          if (ka >= nhi || ka < nlo) sA[v] = -INFINITY;
          if (kb >= nhi || kb < nlo) sB[v] = -INFINITY;
        }
      }
      float bm = fmaxf(fmaxf(fmaxf(sA[0], sA[1]), fmaxf(sA[2], sA[3])), fmaxf(fmaxf(sB[0], sB[1]), fmaxf(sB[2], sB[3])));
      bm = xor16_max(bm);
      bm = xor32_max(bm);
      const float mn = fmaxf(m, bm);
      if (__any((mn - m) * c > 8.f)) {                       // move the max (and rescale) lazily
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - mn) * c);
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) O[tt] *= alpha;
      }
      const float mc = (m == -INFINITY) ? 0.f : m * c;       // a column that has seen no key yet: p = 0
      f16x8 pb;
      float ps = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pa = fast_exp2(fmaf(sA[v], c, -mc));
        const float pv = fast_exp2(fmaf(sB[v], c, -mc));
        ps += pa + pv;
        pb[v] = (_Float16)pa;
        pb[4 + v] = (_Float16)pv;
      }
      lsum += ps;
      const char* vw = kw + UB;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const i32x2 x = lds_read_tr8(vw + tr_off[tt]);
        O[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_f16((uint32_t)x[0], (uint32_t)x[1]), pb, O[tt], 0, 0, 0);
      }
    };
    using Full = std::integral_constant<bool, false>;
    using Edge = std::integral_constant<bool, true>;
    const int edge_hi = min(k1, ctx + 1);                    // units reaching past this need masking,
    auto edge = [&](int u) {                                 // and so do units starting before lo_max
      const int base = (kb0 + 2 * u) * kBlock;
      return base + 2 * kBlock > edge_hi || base < lo_max;
    };

    // one unit in flight while the previous one is computed.  Per wave: the wait leaves exactly the
    // next unit's NCP copies outstanding (vector memory operations complete in issue order).  Whole
    // rows: the wait covers this wave's copies of unit u (and its Q loads), the barrier every wave's,
    // and after it no wave still reads unit u - 1, whose slot the next copies fill.
    issue(0, 0);
    if (live) load_q();
    for (int u = 0; u < nu; ++u) {
      if constexpr (ROWS) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (u + 1 < nu) issue(u + 1, (u + 1) & 1);
      } else if (u + 1 < nu) {
        issue(u + 1, (u + 1) & 1);
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCP) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      if (live) {
        if (edge(u)) consume(Edge{}, u, u & 1);
        else consume(Full{}, u, u & 1);
      }
    }
    lsum = xor16_sum(lsum);
    lsum = xor32_sum(lsum);

    if (on && live) {
      // O^T rows held by this lane are channels 16tt + 4grp + v: apply their V scale
      const float* vsp = a.v_scale + (int64_t)g * D + 4 * grp;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const float4 s = *reinterpret_cast<const float4*>(vsp + 16 * tt);
        O[tt][0] *= s.x;
        O[tt][1] *= s.y;
        O[tt][2] *= s.z;
        O[tt][3] *= s.w;
      }
      if (n_splits == 1) {
        const float inv = 1.f / lsum;
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(t + cr) * a.num_q_heads + h) * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          uint2 pk;
          pk.x = pack_bf16x2(O[tt][0] * inv, O[tt][1] * inv);
          pk.y = pack_bf16x2(O[tt][2] * inv, O[tt][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * tt + 4 * grp) = pk;
        }
      } else {
        const int64_t pidx = partial_index(a, row, cr, split, h);
        float* po = a.part_o + pidx * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          *reinterpret_cast<float4*>(po + 16 * tt + 4 * grp) = make_float4(O[tt][0], O[tt][1], O[tt][2], O[tt][3]);
        if (grp == 0) {
          a.part_ml[pidx * 2] = m * c;     // log2 units
          a.part_ml[pidx * 2 + 1] = lsum;
        }
      }
    }
  };

  // This workgroup's passes: one (row, split), or in stream mode one per row that run pw meets.
  int pw = 0, run_len = 1, gb = 0, gend = 1;
  if constexpr (STREAM) {
    pw = blockIdx.x / nz;
    int unused0, unused1;
    const int tot = stream_scan(a, -1, unused0, unused1);
    run_len = stream_run(a, tot);
    if ((int64_t)pw * run_len >= tot) return;
    gb = pw * run_len;
    gend = (int)min<int64_t>((int64_t)gb + run_len, tot);
  }
  BlockCursor cur;
  while (gb < gend) {
    int row, split, n_splits, b, t, n_keys, ql, k0, k1;
    if constexpr (STREAM) {
      int pre, nbr;
      if (!cur.seek(a, gb, row, pre, nbr)) break;
      const int seg_end = min(gend, pre + nbr);
      resolve_row(a, row, b, t, n_keys, ql);             // a row with blocks on this pass
      const int kbeg = split_origin(a, n_keys, ql);
      k0 = kbeg + kBlock * (gb - pre);
      k1 = min(kbeg + kBlock * (seg_end - pre), n_keys);
      split = pw - pre / run_len;                          // this piece's index among the row's
      n_splits = stream_pieces(pre, nbr, run_len);
      gb = seg_end;
      if constexpr (ROWS) __syncthreads();                 // no wave still reads the last pass's slots
    } else {
      gb = gend;
      const int ib = blockIdx.x / nz;
      split = ib % a.max_splits;
      row = ib / a.max_splits;
      if (row >= a.num_rows || !resolve_row(a, row, b, t, n_keys, ql)) return;
      const int kbeg = split_origin(a, n_keys, ql);
      k0 = kbeg + split * a.split;
      if (k0 >= n_keys) return;
      k1 = min(k0 + a.split, n_keys);
      n_splits = (n_keys - kbeg + a.split - 1) / a.split;
    }
    pass(row, b, t, n_keys, ql, k0, k1, split, n_splits);
  }
}

namespace {
constexpr int kI8WholeRowBytes = 4096;      // cache token rows this wide or wider: whole-row staging

template <int D, int NW, bool ROWS>
hipError_t i8_dispatch(const DecodeArgs& a, hipStream_t s) {
  if (a.heads_per_wg < 1 || a.heads_per_wg > 16) return hipErrorInvalidValue;   // 16 MFMA columns
  const int64_t nzh = ((int64_t)a.qmax * a.group + a.heads_per_wg - 1) / a.heads_per_wg;
  const int64_t per_group = a.stream_wgs > 0 ? (int64_t)a.stream_wgs : (int64_t)a.max_splits * a.num_rows;
  const int64_t grid = (int64_t)((a.num_kv_heads + NW - 1) / NW) * nzh * per_group;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.stream_wgs > 0) decode_i8_kernel<D, NW, ROWS, true><<<dim3((unsigned)grid), dim3(64 * NW), 0, s>>>(a);
  else decode_i8_kernel<D, NW, ROWS, false><<<dim3((unsigned)grid), dim3(64 * NW), 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

// Four waves per workgroup: eight (one workgroup per CU at this register count) measured slower,
// with either staging form.  Whole-row staging where a cache token row holds 4 KiB or more.
hipError_t launch_decode_split_i8(const DecodeArgs& a, int head_dim, hipStream_t s) {
  const bool rows = (int64_t)a.num_kv_heads * head_dim >= kI8WholeRowBytes;
  if (head_dim == 128) return rows ? i8_dispatch<128, 4, true>(a, s) : i8_dispatch<128, 4, false>(a, s);
  if (head_dim == 64) return rows ? i8_dispatch<64, 4, true>(a, s) : i8_dispatch<64, 4, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
