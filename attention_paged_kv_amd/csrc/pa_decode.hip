// pa_decode.hip -- split-KV attention for decode rows (and rows of a few tokens to verify), and the
// cross-split merge.
//
// A decode step reads every cached key and value of its request once (P3 §3.1-3.2, §6.3): the
// pass is bound by HBM bandwidth, not arithmetic.  Work unit = (query row, KV heads and their
// query heads, split of `split` keys).  Each K/V row of a KV head is loaded once and used for all
// the query heads it serves (grouped-query sharing, P3 §2.3), with an online softmax over the
// split's 16-key blocks; the splits of one row are merged by a second kernel with
//   m = max_s m_s,  l = sum_s 2^(m_s - m) l_s,  o = sum_s 2^(m_s - m) o_s / l
// (scores are kept in log2 units: x * scale * log2 e).  The pages do not describe how partial
// softmaxes combine; this is the exact decomposition of the row softmax of P3 §3.1.
// Batches whose rows may carry several positions (tokens to verify) are instead dealt out in
// equal runs of blocks across all rows (stream mode, pa_rows.h); a run's piece of a row is merged
// exactly like a split.
//
// bf16 caches: matrix cores do the arithmetic so that the vector ALUs stay idle however many
// query heads share a KV head.  A workgroup's four waves own four adjacent KV heads; per 16-key
// block and wave (K and V copied into a per-wave LDS slot by direct global->LDS loads):
//   S^T (16 keys x 16 columns) = K (16 x d) . Q^T       -- v_mfma_f32_16x16x32_bf16, K read back
//                                                          from LDS as A operands
//   O^T (d x 16 columns) += V^T (d x 16 keys) . P^T     -- v_mfma_f32_16x16x16_bf16, V read back
//       transposed with ds_read_b64_tr_b16
// P^T stays in registers: the S^T accumulator layout (lane = head, 4 keys) is exactly the B
// operand layout of the second product.  Unused head columns are zero.
// fp32 caches: vector-ALU kernel (dot products reduced across 16-lane rows with DPP; the four
// waves of a workgroup take every 4th block of the split and are merged at the end), serving
// every query row of an fp32 batch.
#include <cstdlib>
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_rows.h"

namespace pa {

namespace {

__device__ __forceinline__ float wave_max_over_groups(float v, int lpr) {
  for (int o = lpr; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_over_groups(float v, int lpr) {
  for (int o = lpr; o < kWave; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool BF16>
struct Io;

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

struct Unit {
  int row, b, t, n_keys, lo, split, k0, k1, n_splits, g, h0, ncols;
};

// Decode the workgroup index into its unit.  Head-group index is fastest so that neighbouring
// workgroups read neighbouring runs of the same token rows.
__device__ __forceinline__ bool get_unit(const DecodeArgs& a, int nzh, Unit& u) {
  const int nz = a.num_kv_heads * nzh;
  int i = blockIdx.x;
  const int z = i % nz;
  i /= nz;
  u.split = i % a.max_splits;
  u.row = i / a.max_splits;
  if (u.row >= a.num_rows) return false;
  int ql;
  if (!resolve_row(a, u.row, u.b, u.t, u.n_keys, ql)) return false;   // per-token rows: ql == 1
  u.lo = first_visible(a, u.n_keys);
  const int kbeg = u.lo & ~(kBlock - 1);
  u.k0 = kbeg + u.split * a.split;
  if (u.k0 >= u.n_keys) return false;
  u.k1 = min(u.k0 + a.split, u.n_keys);
  u.n_splits = (u.n_keys - kbeg + a.split - 1) / a.split;
  u.g = z / nzh;
  const int zh = z % nzh;
  u.h0 = u.g * a.group + zh * a.heads_per_wg;
  u.ncols = min(a.heads_per_wg, a.group - zh * a.heads_per_wg);
  return true;
}

}  // namespace

// ------------------------------------------------------------------------------------------
// bf16: matrix-core split kernel.  A workgroup covers NW adjacent KV heads of the same request
// and split (one wave each), so together its waves read contiguous NW x 256-byte spans of every
// token row.  NW = 4 with two waves per SIMD (two workgroups, eight waves per CU), or, on grids of
// at least two chip-wide rounds and always in stream mode, NW = 2 with one wave per SIMD (two
// workgroups, four waves per CU, each wave with the whole register file).  Measured on this chip: the two-wave form with half the
// copies in flight per CU is faster on such grids (c2 200-201 against 205 us, c5 169 against 174),
// and neither more waves per CU nor spill-free registers alone gave it; on grids of about one round
// the four-wave form is faster (c5 under a 4096-key window 43 against 46 us).  Stream mode (rows of
// tokens to verify, balanced runs) gains on every grid: c5 verifying 4 tokens 167 against 183 us,
// c2 209 against 217, the windowed c5 48 against 50.  Each wave streams all blocks of the split for its head: K and V of a
// block are copied by direct global->LDS loads into one slot of a per-wave double buffer while the
// wave computes on the other slot (rows' 16-byte chunks XOR-swizzled so the K operand reads and the
// V transpose reads are free of bank conflicts).  The copies are issued as inline assembly and
// waited for with explicit vmcnt counts: with direct-to-LDS loads in view, the compiler waits for
// every outstanding copy before an LDS read, which would wait for the next block's copies before
// the current block is computed and leave no load in flight during the arithmetic.  The MFMA
// columns are (position, query head) pairs of the request: a decode row has one position, a row of
// a few tokens to verify (P4 "一步的 token 预算": speculative verification advances several tokens in
// one step) has q_len of them, each masked to its own causal (and window) range, so the K/V of the
// request are read once for all of them.  Unused columns are zero.
// ------------------------------------------------------------------------------------------
namespace {
// Physical 16-byte chunk of logical chunk q in staged V row r is q ^ dswz<D>(r): a permutation of the
// row's D/8 chunks that keeps the transpose reads of a wave on distinct LDS banks.
template <int D>
__device__ __forceinline__ int dswz(int r) {
  if constexpr (D == 128) return 2 * (r & 7);
  else return (((r ^ (r >> 2)) & 1) << 1) | (((r >> 1) & 1) << 2);
}
// Same for staged K rows, read as 16-byte A operands by lanes (row = lane % 16, chunk 4kk + lane / 16):
// the 16 rows of one 16-lane group land on 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}
}

// A row with more than 16 (position, head) columns (several tokens to verify on a grouped-query
// model, or more than 16 query heads per KV head) carries two column groups of 16 through each pass
// over the split's keys, so K and V are read once for 32 columns; the choice is made per workgroup
// from its own row, and both forms are compiled into the kernel.
template <int D, bool STREAM, int NW>
__global__ __launch_bounds__(64 * NW, NW == 2 ? 1 : 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NKK = D / 32;                 // 16x16x32 k-steps over d for S^T
  constexpr int NT = D / 16;                  // 16-row d tiles of O^T
  constexpr int ROWB = D * 2;                 // bytes of one head's K or V row
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per wave-wide 1 KiB copy
  constexpr int IPB = kBlock / RPI;           // copies per 16-row block
  constexpr int VB = kBlock * ROWB;           // bytes per staged K (or V) block
  constexpr int NCP = 2 * IPB;                // copies per block (K and V)
  __shared__ __align__(16) char sKV[2 * NW * 2 * VB];  // [slot][wave][K block, V block]

  // unit: (row, split) -- or, in stream mode, run pw of the concatenated blocks of all rows, taken
  // as one piece per row it meets -- for head group `quad` of NW KV heads (fastest); the wave's KV
  // head is NW * quad + w.  A row with more (position, head) columns than NG MFMAs hold runs its column
  // groups NG at a time in the same workgroup (the K/V re-read comes straight after the first pass).
  const int nq = (a.num_kv_heads + NW - 1) / NW;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = blockIdx.x % nq;
  const int g = NW * quad + w;
  if (g >= a.num_kv_heads) return;                         // waves are independent: no barriers
  int row, split, b, t0, n_keys, ql, ctx, lo_min, lo_max, k0, k1, n_splits, ncol_all;

  auto run = [&](auto ng_tag) {
    constexpr int NG = decltype(ng_tag)::value;
    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15;                  // S^T / O^T column; also the K row read
    const int grp = lane >> 4;                  // 4-key group of the accumulator layout
    const float c = a.scale_log2;

    const int64_t rs = (int64_t)a.num_kv_heads * D;            // elements per cache token row
    const int64_t blkbytes = kBlock * rs * 2;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * ROWB;
    const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;
    const int kb0 = k0 / kBlock;
    const int nb = (k1 + kBlock - 1) / kBlock - kb0;
    int ids = 0, ids_base = -kWave;                            // lane i: id of block ids_base + i

    // K operand: key row `col`, d = 32kk + 8grp, i.e. logical chunk 4kk + grp of the staged row
    uint32_t k_rd[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) k_rd[kk] = col * ROWB + (((4 * kk + grp) ^ kswz<D>(col)) * 16);
    // copies: copy i covers rows RPI*i ..; lane -> (row RPI*i + lane / CPR, physical chunk lane % CPR),
    // which holds logical chunk (lane % CPR) ^ swz(row) of the cache row
    uint32_t k_lane[IPB], v_lane[IPB];
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int r = RPI * i + lane / CPR;
      k_lane[i] = (uint32_t)(r * rs * 2) + (((lane % CPR) ^ kswz<D>(r)) * 16);
      v_lane[i] = (uint32_t)(r * rs * 2) + (((lane % CPR) ^ dswz<D>(r)) * 16);
    }
    // transpose read: group grp, lane j = 4e + cq reads row 4grp + e, columns 16tt + 4cq .. +3,
    // i.e. logical chunk 2tt + cq / 2, byte half cq & 1
    uint32_t tr_off[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int r = 4 * grp + (col >> 2);
      const int lq = 2 * tt + ((col & 3) >> 1);
      tr_off[tt] = r * ROWB + ((lq ^ dswz<D>(r)) * 16) + (col & 1) * 8;
    }

    char* const mine = sKV + w * 2 * VB;                       // this wave's slot 0; slot 1 is 2NW * VB on
    auto issue = [&](int i, int slot) {                        // block kb0 + i: K and V into the slot
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      // the slot's earlier reads are done
      if (i - ids_base >= kWave) {                             // next 64 ids (once per 64 blocks)
        ids_base = i;
        ids = load_ids_sync(table + kb0 + i, nb - i);
      }
      const char* kb = kbase + (int64_t)__builtin_amdgcn_readlane(ids, i - ids_base) * blkbytes;
      const char* vb = vbase + (kb - kbase);
      const uint32_t l = __builtin_amdgcn_readfirstlane(lds_u32(mine + slot * 2 * NW * VB));
#pragma unroll
      for (int j = 0; j < IPB; ++j) dma16(kb, k_lane[j], l + 1024 * j);
#pragma unroll
      for (int j = 0; j < IPB; ++j) dma16(vb, v_lane[j], l + VB + 1024 * j);
    };

    for (int zh = 0; zh * a.heads_per_wg < ncol_all; zh += NG) {
      issue(0, 0);                              // the first block's copies overlap the Q loads
      // this pass's columns: group gi holds columns (zh + gi) * heads_per_wg + col
      bool on[NG];
      int cr[NG], h[NG], nvis[NG], lo_c[NG];
      bf16x8 qb[NG][NKK];                       // Q^T as the B operand: d = 32kk + 8grp .. +8
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int c0 = (zh + gi) * a.heads_per_wg;
        on[gi] = col < min(a.heads_per_wg, ncol_all - c0);
        cr[gi] = on[gi] ? (c0 + col) / a.group : 0;            // this column's position in the request
        h[gi] = g * a.group + (on[gi] ? (c0 + col) % a.group : 0);
        nvis[gi] = ctx + cr[gi] + 1;                           // keys [lo_c, nvis) are this column's
        lo_c[gi] = first_visible(a, nvis[gi]);
        const char* qp = reinterpret_cast<const char*>(a.q) +
                         (((int64_t)(t0 + cr[gi]) * a.num_q_heads + h[gi]) * D + 8 * grp) * 2;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const uint4 v = on[gi] ? *reinterpret_cast<const uint4*>(qp + kk * 64) : make_uint4(0, 0, 0, 0);
          qb[gi][kk] = __builtin_bit_cast(bf16x8, v);
        }
      }
      // wait for Q (and the first block) here: left to itself the compiler may put this wait (a
      // full vmcnt(0)) inside the block loop, where it would also wait for the next block
      __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0) only

      float m[NG], lsum[NG];
      floatx4 O[NG][NT];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        m[gi] = -INFINITY;
        lsum[gi] = 0.f;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) O[gi][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }

      // one block.  EDGE blocks hold keys some column must not see -- before its window or after its
      // position (the split's last blocks, and the first blocks of split 0 under a window).  The
      // test is uniform across the wave and picks one of two compiled copies, so other blocks carry
      // no masking at all.
      auto consume_as = [&](auto edge_tag, int i, int slot) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        const int s0 = (kb0 + i) * kBlock;
        const char* kw = mine + slot * 2 * NW * VB;
        bf16x8 kop[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) kop[kk] = *reinterpret_cast<const bf16x8*>(kw + k_rd[kk]);
        bf16x4 pb[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kk], qb[gi][kk], sc, 0, 0, 0);
          if constexpr (EDGE) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int key = s0 + 4 * grp + v;
              if (key >= nvis[gi] || key < lo_c[gi]) sc[v] = -INFINITY;
            }
          }
          float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
          bm = xor16_max(bm);
          bm = xor32_max(bm);
          const float mn = fmaxf(m[gi], bm);
          const float alpha = (m[gi] == -INFINITY) ? 0.f : fast_exp2((m[gi] - mn) * c);
          const float mc = (mn == -INFINITY) ? 0.f : mn * c;   // a column with no key yet: p = 0
          float p[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) p[v] = fast_exp2(fmaf(sc[v], c, -mc));
          lsum[gi] = lsum[gi] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
          m[gi] = mn;
#pragma unroll
          for (int v = 0; v < 4; ++v) pb[gi][v] = (__bf16)p[v];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) O[gi][tt] *= alpha;
        }
        const char* vw = kw + VB;
        bf16x4 vt[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) vt[tt] = lds_read_tr(reinterpret_cast<const uint16_t*>(vw + tr_off[tt]));
        if constexpr (EDGE) {
          // rows no column may see (before the first window, past the last position) may hold poison
          // under p = 0: zero them
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = s0 + 4 * grp + e;
              if (key >= n_keys || key < lo_min) vt[tt][e] = (__bf16)0.f;
            }
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            O[gi][tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[tt], pb[gi], O[gi][tt], 0, 0, 0);
      };
      auto consume = [&](int i, int slot) {
        const int s0 = (kb0 + i) * kBlock;
        if (s0 < lo_max || s0 + kBlock > ctx + 1) consume_as(std::true_type{}, i, slot);
        else consume_as(std::false_type{}, i, slot);
      };

      // one block in flight while the previous one is computed; the wait leaves exactly the next
      // block's NCP copies outstanding (vector memory operations complete in issue order)
      for (int i = 0; i < nb; ++i) {
        if (i + 1 < nb) {
          issue(i + 1, (i + 1) & 1);
          asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCP) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        consume(i, i & 1);
      }

      // this wave holds the whole split for its head: write each column's row or the split's partial
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        float ls = xor16_sum(lsum[gi]);
        ls = xor32_sum(ls);
        if (!on[gi]) continue;
        if (n_splits == 1) {
          const float inv = 1.f / ls;
          uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(t0 + cr[gi]) * a.num_q_heads + h[gi]) * D;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            uint2 pk;
            pk.x = pack_bf16x2(O[gi][tt][0] * inv, O[gi][tt][1] * inv);
            pk.y = pack_bf16x2(O[gi][tt][2] * inv, O[gi][tt][3] * inv);
            *reinterpret_cast<uint2*>(op + 16 * tt + 4 * grp) = pk;
          }
        } else {
          const int64_t pidx = partial_index(a, row, cr[gi], split, h[gi]);
          float* po = a.part_o + pidx * D;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            *reinterpret_cast<float4*>(po + 16 * tt + 4 * grp) =
                make_float4(O[gi][tt][0], O[gi][tt][1], O[gi][tt][2], O[gi][tt][3]);
          if (grp == 0) {
            a.part_ml[pidx * 2] = m[gi] * c;     // log2 units
            a.part_ml[pidx * 2 + 1] = ls;
          }
        }
      }
    }
  };
  // row fields the unit needs, once (row, keys [k0, k1), piece index and count) are set
  auto setup = [&]() {
    resolve_row(a, row, b, t0, n_keys, ql);
    ctx = n_keys - ql;                                     // keys before the request's first position
    lo_min = first_visible(a, ctx + 1);                    // oldest key any position sees
    lo_max = first_visible(a, n_keys);                     // oldest key the last position sees
    ncol_all = ql * a.group;                               // (position, head) columns of the row
  };
  auto go = [&]() {
    if (ncol_all > a.heads_per_wg) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  };
  if constexpr (STREAM) {
    const int pw = blockIdx.x / nq;
    int unused0, unused1;
    const int tot = stream_scan(a, -1, unused0, unused1);
    const int run_len = stream_run(a, tot);
    if ((int64_t)pw * run_len >= tot) return;
    const int gbeg = pw * run_len;
    const int gend = (int)min<int64_t>((int64_t)gbeg + run_len, tot);
    BlockCursor cur;
    for (int gb = gbeg; gb < gend;) {
      int pre, nbr;
      if (!cur.seek(a, gb, row, pre, nbr)) break;
      const int seg_end = min(gend, pre + nbr);
      setup();
      const int kbeg = lo_min & ~(kBlock - 1);
      k0 = kbeg + kBlock * (gb - pre);
      k1 = min(kbeg + kBlock * (seg_end - pre), n_keys);
      split = pw - pre / run_len;                          // this piece's index among the row's
      n_splits = stream_pieces(pre, nbr, run_len);
      gb = seg_end;
      go();
    }
  } else {
    const int ib = blockIdx.x / nq;
    split = ib % a.max_splits;
    row = ib / a.max_splits;
    if (row >= a.num_rows) return;
    int b_, t_, n_, q_;
    if (!resolve_row(a, row, b_, t_, n_, q_)) return;
    setup();
    const int kbeg = lo_min & ~(kBlock - 1);
    k0 = kbeg + split * a.split;
    if (k0 >= n_keys) return;
    k1 = min(k0 + a.split, n_keys);
    n_splits = (n_keys - kbeg + a.split - 1) / a.split;
    go();
  }
}

// ------------------------------------------------------------------------------------------
// Vector-ALU split kernel for fp32 caches.  GT query heads per workgroup (GT divides the group
// size).  Each K/V row is read by a row group of lanes with 16-byte loads; q.k is reduced across the
// group with DPP, and every row group keeps its own running max / sum / accumulator.
// ------------------------------------------------------------------------------------------
template <int D, int GT, bool BF16>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using IO = Io<BF16>;
  constexpr int EPL = IO::kEpl;
  constexpr int LPR = D * IO::kEsz / 16;     // lanes per K/V row
  constexpr int RPL = kWave / LPR;           // rows per wave-wide load
  constexpr int LPB = kBlock / RPL;          // loads per 16-key block
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row width");

  __shared__ float sm_m[4][GT];
  __shared__ float sm_l[4][GT];
  __shared__ float sm_o[4][GT][D];

  Unit u;
  if (!get_unit(a, a.group / GT, u)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int rg = lane / LPR;                 // row group within the wave
  const int cl = lane % LPR;                 // which 16-byte piece of the row

  float qf[GT][EPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    const int64_t qoff = ((int64_t)u.t * a.num_q_heads + u.h0 + hh) * D + cl * EPL;
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
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + ((int64_t)u.g * D + cl * EPL) * IO::kEsz;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + ((int64_t)u.g * D + cl * EPL) * IO::kEsz;
  const int32_t* table = a.block_tables + (int64_t)u.b * a.max_blocks;
  const int kb0 = u.k0 / kBlock;
  const int kb1 = (u.k1 + kBlock - 1) / kBlock;

  const int nw = (kb1 - kb0 - w + 3) / 4;             // blocks this wave visits: kb0 + w + 4i
  BlockWindow win;
  auto load_block = [&](int blk, uint4* kr, uint4* vr) {
    const int64_t base = (int64_t)win.get(table, kb0 + w, 4, nw, (blk - kb0 - w) >> 2) * kBlock * rs;
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
    const bool full = (blk + 1) * kBlock <= u.k1 && blk * kBlock >= u.lo;
    float vf[LPB][EPL];
#pragma unroll
    for (int r = 0; r < LPB; ++r) {
      IO::widen(vr[r], vf[r]);
      if (!full && (key0 + r * RPL >= u.k1 || key0 + r * RPL < u.lo)) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[r][e] = 0.f;      // slots outside [lo, k1)
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
    const int h = u.h0 + hh;
    if (u.n_splits == 1) {
      IO::store(a.out, ((int64_t)u.t * a.num_q_heads + h) * D + dd, o / ll);
    } else {
      const int64_t pidx = partial_index(a, u.row, 0, u.split, h);
      a.part_o[pidx * D + dd] = o;
      if (dd == 0) {
        a.part_ml[pidx * 2] = mm;
        a.part_ml[pidx * 2 + 1] = ll;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Cross-split merge: one workgroup per (row, position, query head).  Groups of its threads each fold
// a share of the splits in one pass (a running max, their partials read together), and the groups
// are then combined in LDS: one round of reads instead of a max pass, a sum pass and an output pass.
// ------------------------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int CH = D / 4;                  // float4 chunks of a row
  constexpr int NG = 256 / CH;               // split groups
  __shared__ float4 racc[NG][CH];
  __shared__ float sm[NG], sl[NG];

  const int h = blockIdx.x % a.num_q_heads;
  const int r = (blockIdx.x / a.num_q_heads) % a.qmax;
  const int row = blockIdx.x / (a.num_q_heads * a.qmax);
  int b, t0, n_keys, ql;
  if (!resolve_row(a, row, b, t0, n_keys, ql) || r >= ql) return;
  const int t = t0 + r;
  int n;
  if (a.stream_wgs > 0) {
    int pre, nb;
    const int tot = stream_scan(a, row, pre, nb);
    n = stream_pieces(pre, nb, stream_run(a, tot));
  } else {
    n = (n_keys - split_origin(a, n_keys, ql) + a.split - 1) / a.split;
  }
  if (n <= 1) return;                                       // written directly by the split kernel
  const int tid = threadIdx.x;
  const int64_t pbase = partial_index(a, row, r, 0, h);    // split s adds s * num_q_heads
  const float* ml = a.part_ml;

  // one pass: group g folds splits g, g + NG, ... into (m, l, o) with a running max (all threads
  // of a group see the same splits, so the same m and l), then the groups are combined in LDS
  const int cidx = tid % CH, gidx = tid / CH;
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = gidx; s < n; s += NG) {
    const int64_t p = pbase + (int64_t)s * a.num_q_heads;
    const float ms = ml[p * 2], ls = ml[p * 2 + 1];
    const float4 o = reinterpret_cast<const float4*>(a.part_o + p * D)[cidx];
    const float mn = fmaxf(m, ms);
    const float wo = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);   // weight of what is folded so far
    const float ws = (ms == -INFINITY) ? 0.f : fast_exp2(ms - mn); // a split that saw no key: 0
    l = fmaf(ls, ws, l * wo);
    acc.x = fmaf(o.x, ws, acc.x * wo);
    acc.y = fmaf(o.y, ws, acc.y * wo);
    acc.z = fmaf(o.z, ws, acc.z * wo);
    acc.w = fmaf(o.w, ws, acc.w * wo);
    m = mn;
  }
  racc[gidx][cidx] = acc;
  if (cidx == 0) {
    sm[gidx] = m;
    sl[gidx] = l;
  }
  __syncthreads();
  if (tid < CH) {
    float M = sm[0];
#pragma unroll
    for (int g = 1; g < NG; ++g) M = fmaxf(M, sm[g]);
    float4 rr = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (sm[g] == -INFINITY) continue;                     // a group with no split (n < NG)
      const float wg = fast_exp2(sm[g] - M);
      const float4 x = racc[g][tid];
      L = fmaf(sl[g], wg, L);
      rr.x = fmaf(x.x, wg, rr.x);
      rr.y = fmaf(x.y, wg, rr.y);
      rr.z = fmaf(x.z, wg, rr.z);
      rr.w = fmaf(x.w, wg, rr.w);
    }
    const float inv = 1.f / L;
    const int64_t o = ((int64_t)t * a.num_q_heads + h) * D + 4 * tid;
    if (BF16) {
      uint2 pk;
      pk.x = pack_bf16x2(rr.x * inv, rr.y * inv);
      pk.y = pack_bf16x2(rr.z * inv, rr.w * inv);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o) = pk;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o) =
          make_float4(rr.x * inv, rr.y * inv, rr.z * inv, rr.w * inv);
    }
  }
}

// Merge for stream mode, where a row has few pieces: one wave per (row, position, query head), four
// per workgroup, no LDS.  The wave's lanes are 4 piece groups x 16 channel chunks; each piece's
// weight 2^(m_s - m) is recomputed where it is used, so one pass over the partials suffices after
// the max.  (With fixed splits a long row has dozens of partials; there a workgroup per item reads
// them in parallel, above, and measured faster.)
template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_wave_kernel(DecodeArgs a) {
  constexpr int CL = D / 16;                 // channels per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = (int)(item % a.num_q_heads);
  const int r = (int)((item / a.num_q_heads) % a.qmax);
  const int64_t row64 = item / ((int64_t)a.num_q_heads * a.qmax);
  if (row64 >= a.num_rows) return;
  const int row = (int)row64;
  int b, t0, n_keys, ql;
  if (!resolve_row(a, row, b, t0, n_keys, ql) || r >= ql) return;
  int n;
  if (a.stream_wgs > 0) {
    int pre, nb;
    const int tot = stream_scan(a, row, pre, nb);
    n = stream_pieces(pre, nb, stream_run(a, tot));
  } else {
    n = (n_keys - split_origin(a, n_keys, ql) + a.split - 1) / a.split;
  }
  if (n <= 1) return;                                       // written directly by the split kernel
  const int64_t pbase = partial_index(a, row, r, 0, h);    // split s adds s * num_q_heads
  const int64_t st = a.num_q_heads;
  const float* ml = a.part_ml;

  float mx = -INFINITY, ls = 0.f;
  for (int s = lane; s < n; s += kWave) mx = fmaxf(mx, ml[(pbase + s * st) * 2]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  for (int s = lane; s < n; s += kWave) {
    const float* p = ml + (pbase + s * st) * 2;
    ls = fmaf(fast_exp2(p[0] - mx), p[1], ls);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);

  const int sg = lane >> 4, ch = lane & 15;                 // split group, channel chunk
  float acc[CL];
#pragma unroll
  for (int e = 0; e < CL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int s0 = 0; s0 < n; s0 += 4) {
    const int s = s0 + sg;
    if (s < n) {
      const int64_t p = pbase + s * st;
      const float wgt = fast_exp2(ml[p * 2] - mx);
      const float4* o = reinterpret_cast<const float4*>(a.part_o + p * D + CL * ch);
#pragma unroll
      for (int e4 = 0; e4 < CL / 4; ++e4) {
        const float4 v = o[e4];
        acc[4 * e4] = fmaf(wgt, v.x, acc[4 * e4]);
        acc[4 * e4 + 1] = fmaf(wgt, v.y, acc[4 * e4 + 1]);
        acc[4 * e4 + 2] = fmaf(wgt, v.z, acc[4 * e4 + 2]);
        acc[4 * e4 + 3] = fmaf(wgt, v.w, acc[4 * e4 + 3]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < CL; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (sg == 0) {
    const float inv = 1.f / ls;
    const int64_t o = ((int64_t)(t0 + r) * a.num_q_heads + h) * D + CL * ch;
    if constexpr (BF16) {
#pragma unroll
      for (int e2 = 0; e2 < CL / 2; ++e2)
        reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + o)[e2] =
            pack_bf16x2(acc[2 * e2] * inv, acc[2 * e2 + 1] * inv);
    } else {
#pragma unroll
      for (int e4 = 0; e4 < CL / 4; ++e4)
        reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o)[e4] =
            make_float4(acc[4 * e4] * inv, acc[4 * e4 + 1] * inv, acc[4 * e4 + 2] * inv, acc[4 * e4 + 3] * inv);
    }
  }
}

// ------------------------------------------------------------------------------------------
namespace {
template <int D>
hipError_t mfma_dispatch(const DecodeArgs& a, dim3 g, hipStream_t s) {
  if (a.heads_per_wg < 1 || a.heads_per_wg > 16) return hipErrorInvalidValue;   // 16 MFMA columns
  if (a.stream_wgs > 0) decode_mfma_kernel<D, true, 2><<<g, dim3(128), 0, s>>>(a);
  else if (a.pair_wgs) decode_mfma_kernel<D, false, 2><<<g, dim3(128), 0, s>>>(a);
  else decode_mfma_kernel<D, false, 4><<<g, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}
template <int D, bool BF16>
hipError_t valu_dispatch(const DecodeArgs& a, dim3 g, hipStream_t s) {
  const dim3 blk(256);
  switch (a.heads_per_wg) {
    case 1: decode_valu_kernel<D, 1, BF16><<<g, blk, 0, s>>>(a); break;
    case 2: decode_valu_kernel<D, 2, BF16><<<g, blk, 0, s>>>(a); break;
    case 4: decode_valu_kernel<D, 4, BF16><<<g, blk, 0, s>>>(a); break;
    case 8: decode_valu_kernel<D, 8, BF16><<<g, blk, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s) {
  const int64_t nzh = ((int64_t)a.qmax * a.group + a.heads_per_wg - 1) / a.heads_per_wg;
  const int nw = (a.stream_wgs > 0 || a.pair_wgs) ? 2 : 4;                     // MFMA: KV heads per WG
  const int64_t heads = bf16 ? (a.num_kv_heads + nw - 1) / nw : a.num_kv_heads;
  // MFMA: one workgroup per (row, split) or stream_wgs runs, per group of nw KV heads, column groups looping
  // inside the workgroup; fp32: one workgroup per (row, split, column group)
  const int64_t grid = bf16 ? heads * (a.stream_wgs > 0 ? a.stream_wgs : a.max_splits * a.num_rows)
                            : heads * nzh * a.max_splits * a.num_rows;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid);
  if (bf16) {
    if (head_dim == 128) return mfma_dispatch<128>(a, g, s);
    if (head_dim == 64) return mfma_dispatch<64>(a, g, s);
  } else {
    if (head_dim == 128) return valu_dispatch<128, false>(a, g, s);
    if (head_dim == 64) return valu_dispatch<64, false>(a, g, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s) {
  const int64_t items = (int64_t)a.num_rows * a.qmax * a.num_q_heads;
  const bool wave = a.stream_wgs > 0;                      // few pieces per row: a wave per item
  const int64_t grid = wave ? (items + 3) / 4 : items;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(256);
  if (head_dim == 128) {
    if (wave) bf16 ? merge_wave_kernel<128, true><<<g, blk, 0, s>>>(a) : merge_wave_kernel<128, false><<<g, blk, 0, s>>>(a);
    else bf16 ? decode_merge_kernel<128, true><<<g, blk, 0, s>>>(a) : decode_merge_kernel<128, false><<<g, blk, 0, s>>>(a);
  } else if (head_dim == 64) {
    if (wave) bf16 ? merge_wave_kernel<64, true><<<g, blk, 0, s>>>(a) : merge_wave_kernel<64, false><<<g, blk, 0, s>>>(a);
    else bf16 ? decode_merge_kernel<64, true><<<g, blk, 0, s>>>(a) : decode_merge_kernel<64, false><<<g, blk, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
