// pa_prefill.hip -- causal attention tiles for requests with q_len >= 2 (one-shot prefill and
// chunked prefill), on bf16 MFMA.  Each workgroup finds its own tile from its index.
//
// A prefill row block attends over every key up to its own position (P3 §2.1) and a chunk
// additionally reads the keys of all earlier chunks from the cache (P4 "块大小怎样取舍": chunk 15
// reads the KV of the 14 chunks before it).  The S x S score matrix is never stored: K/V tiles are
// staged in LDS and consumed with an online softmax (P3 §2.1, P1 §2.1 describe the on-chip tiling
// idea; the tiling here is CDNA4's own).  Arithmetic intensity is ~S FLOP/byte, so this part is a
// dense contraction and runs on the matrix cores.
//
// Tile shape: 256 query rows x 64 keys per step, eight waves of 32 rows (two per SIMD, one
// workgroup per CU), so each K/V tile staged in LDS serves 256 rows.  A query row is a
// (position, query head) pair; the Hq/Hkv heads of one KV group are packed into the rows of the
// same tile so that each K/V tile is loaded once for the whole group.  Per wave and key tile:
//   S^T (64 keys x 32 rows) = K (64 x d) . Q^T (d x 32)     -- v_mfma_f32_32x32x16_bf16
//   online softmax on S^T in registers (lane = query row, 16 keys per lane and sub-tile)
//   O^T (d x 32 rows)     += V^T (d x 64) . P^T (64 x 32)   -- P^T stays in registers
// K and V tiles are staged in LDS by direct global->LDS loads (no staging registers), double
// buffered: the next tile's loads are in flight while the current one is consumed, with one
// workgroup barrier per tile.  For bf16 caches the copies are issued as inline assembly and waited
// for explicitly, so the compiler's own wait counting stays precise: K operands are then read two
// k-steps ahead of their products instead of being waited for pair by pair.  Each wave loads one 16-key cache block per tile, so its block-table
// lookup is a single uniform value.  LDS rows are unpadded and their 16-byte chunks XOR-swizzled by
// row, which keeps the K operand reads and the V transpose reads free of bank conflicts.  V^T
// operands come from the LDS transpose read: the S^T accumulator layout gives lane half a the keys
// {4a..4a+3, 8+4a..8+4a+3} of each 16-key step, which is exactly two 4-row transpose reads.  Key
// tiles entirely above the causal diagonal of the last row are never visited; only tiles crossing
// the diagonal are masked.  Keys past the request's length in its last tile load a valid row
// instead (finite data under a zero probability).  With a sliding window (P2 §5.2, P3 §6.3: only
// the most recent W keys count) the key loop starts at the tile holding the first row's oldest
// visible key, and tiles crossing the window's lower edge are masked as well; keys older than the
// request's first window are never read (their blocks may be gone), a valid row stands in.
// Scores are in log2 units: Q is multiplied by scale * log2(e) once and rounded to bf16.  Each row
// keeps a reference max m_ref, a bf16 value, and its QK^T products start from -m_ref in the
// accumulators instead of zero, so they give s - m_ref directly and the
// probabilities are exp2 of the accumulators with no vector arithmetic before the exponential.
// The reference is only moved (and O rescaled) when a row with none sees its first key or some
// row's max exceeds it by more than 2^8; between moves, probabilities are at most about 2^8.
//
// 8-bit caches (P2 §4.3, §5.4: int8 codes with a scale per KV head and channel): the cache blocks
// are copied to int8 staging buffers the same way, then the workgroup converts each tile once into
// the bf16 tile layout above (exact: |code| <= 127), so the tile math is unchanged; the K scale is
// folded into the query (q * k_scale rounded to bf16) and the V scale multiplies O at the end.  The
// bf16 tiles are double buffered: tile kt + 1 is converted in the same phase as tile kt's math.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

namespace {
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Physical 16-byte chunk of logical chunk q in tile row r (bijective per row).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return (r >> 1) & 7;
}
}  // namespace

// One int32 per lane, loaded and waited for inside one asm block.  The key loop contains no load
// the compiler can see: a visible load makes it place conservative vmcnt(0) waits in the loop, and
// those would also wait for the next tile's copies (issued as inline assembly, which it does not
// count), serialising the copies with the products.
__device__ __forceinline__ int load_i32_sync(const int32_t* p) {
  int v;
  asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
// Block ids of a wave's blocks, 64 at a time (lane i: the id of block first + stride * (base + i)),
// taken with one v_readlane each; the ids are loaded with load_i32_sync (once per 64 tiles).
// get() is only called for k < count, so count >= 1 and lanes past the end load the last entry.
struct SyncWindow {
  int ids = 0;
  int base = -(1 << 30);
  __device__ __forceinline__ int get(const int32_t* table, int first, int stride, int count, int k) {
    if (k - base >= 64 || k < base) {
      base = k;
      const int i = k + (int)(threadIdx.x & 63);
      ids = load_i32_sync(table + first + stride * min(i, count - 1));
    }
    return __builtin_amdgcn_readlane(ids, k - base);
  }
};

template <int D, bool KV8>
__global__ __launch_bounds__(512, 1) void prefill_tile_kernel(TileArgs a) {
  constexpr int ESZ = KV8 ? 1 : 2;          // bytes per cache element
  constexpr int ROWB = D * 2;               // bytes per bf16 K/V row in LDS
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;          // rows per wave-wide 1 KiB load
  constexpr int IPB = kBlock / RPI;         // loads per 16-key block (per tensor)
  constexpr int TILEB = kTileKeys * ROWB;   // bytes per K (or V) tile
  constexpr int NKK = D / 16;               // MFMA k-steps over d
  constexpr int NDT = D / 32;               // 32-wide d tiles of O^T
  static_assert(kTileKeys == 4 * kBlock, "one cache block per wave and tile");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // slot -> (request b, first local row q_off, rows n_pos): the tiles are the requests' row
  // blocks of pos_per_tile positions, requests in order and each request's last (longest) row
  // block first; requests with q_len < min_q have none.  Every wave finds its slot with a
  // wave-wide prefix sum over the tile counts, 64 requests at a time.
  int b = -1, q_off = 0, n_pos = 0;
  {
    int base = 0;
    for (int c0 = 0; c0 < a.num_seqs; c0 += kWave) {
      const int r = c0 + lane;
      int qlr = 0, cnt = 0;
      if (r < a.num_seqs) {
        qlr = a.qsl[r + 1] - a.qsl[r];
        cnt = qlr >= a.min_q ? (qlr + a.pos_per_tile - 1) / a.pos_per_tile : 0;
      }
      const int incl = wave_incl_scan(cnt);
      const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (slot < base + total) {
        const int j = __popcll(__ballot(incl <= slot - base));   // requests wholly before the slot
        b = c0 + j;
        const int k = slot - base - __builtin_amdgcn_readlane(incl - cnt, j);   // its k-th tile
        const int qi = __builtin_amdgcn_readlane(cnt, j) - 1 - k;                // last block first
        q_off = qi * a.pos_per_tile;
        n_pos = min(a.pos_per_tile, __builtin_amdgcn_readlane(qlr, j) - q_off);
        break;
      }
      base += total;
    }
  }
  if (b < 0) return;                             // past the last tile
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
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + kk * 32) : make_uint4(0, 0, 0, 0);
      // q * scale * log2(e) (and * k_scale for int8 caches), rounded once to bf16: the products are
      // then scores in log2 units
      const float cs = a.scale_log2;
      if constexpr (KV8) {                       // q * k_scale of channels 16kk + 8half .. +7
        const float* ks = a.k_scale + (int64_t)g * D + 16 * kk + 8 * half;
        const float4 s0 = *reinterpret_cast<const float4*>(ks);
        const float4 s1 = *reinterpret_cast<const float4*>(ks + 4);
        const float f[8] = {bf16_lo(v.x) * s0.x, bf16_hi(v.x) * s0.y, bf16_lo(v.y) * s0.z, bf16_hi(v.y) * s0.w,
                            bf16_lo(v.z) * s1.x, bf16_hi(v.z) * s1.y, bf16_lo(v.w) * s1.z, bf16_hi(v.w) * s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[kk][e] = (__bf16)(f[e] * cs);
      } else {
        const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                            bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[kk][e] = (__bf16)(f[e] * cs);
      }
    }
  }

  // wait for Q here: left to itself the compiler puts this wait (vmcnt(0)) inside the key loop,
  // where it would also wait for the next tile's copies
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0) only

  const int kv_end = min(sl, ctx + q_off + n_pos);   // keys needed by the last row of the tile
  const int n_kt = (kv_end + kTileKeys - 1) / kTileKeys;
  const int first_pos = ctx + q_off;
  const int last_pos = kv_end - 1;
  const int lo_req = max(0, ctx - a.window + 1);     // oldest key any row of the request sees
  const int kt_lo = max(0, first_pos - a.window + 1) / kTileKeys;   // first key tile of this tile
  const int low_edge = last_pos - a.window + 1;      // tiles starting below this need the window mask
  const int64_t rs = (int64_t)a.num_kv_heads * D;    // elements per cache token row
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * D * ESZ;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * D * ESZ;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_blocks;

  // staging: waves 0-3 copy the tile's four K blocks, waves 4-7 its four V blocks; wave w takes
  // block 4kt + (w & 3), and those entirely below the length come from a window of table entries
  const int bw = w & 3;
  const bool is_v = w >= 4;
  const char* tbase = is_v ? vbase : kbase;
  const int n_full = (sl / kBlock - bw + 3) / 4;  // count of kt with (4kt + bw + 1) * 16 <= sl
  SyncWindow win;

  // m_ref: the row's reference max (log2 units, rounded to a bf16 value); has_ref: whether the row
  // has one yet (before its first visible key it does not, and m_ref is 0).  The products give
  // s - m_ref directly: both QK^T chains start from mref16, the lane's -m_ref in every accumulator
  // entry (a lane's 16 entries all belong to its own row), instead of from zero.
  float m_ref = 0.f, l_run = 0.f;
  bool has_ref = false;
  floatx16 mref16;
#pragma unroll
  for (int v = 0; v < 16; ++v) mref16[v] = 0.f;
  floatx16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[dt][v] = 0.f;

  // K operand: row 32st + l32, logical chunk 2kk + half.  swz(r) depends on r mod 16 only, so the
  // second sub-tile (rows + 32) is the same offset plus an immediate.
  uint32_t k_off[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) k_off[kk] = l32 * ROWB + (((2 * kk + half) ^ swz<D>(l32)) * 16);
  // V transpose-read coordinates: 16-lane group (gsel, j = 4e + cq) reads row R + e, columns
  // 32dt + 16gsel + 4cq .. +3 (8 bytes), i.e. logical chunk 4dt + 2gsel + cq/2, half cq & 1.
  const int trj = lane & 15;
  const int gsel = (lane >> 4) & 1;
  const int tre = trj >> 2;
  // rows 16kk + 4half + tre (lo) and + 8 (hi): swz of those rows does not depend on kk
  uint32_t v_off[2][NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int lq = 4 * dt + 2 * gsel + (trj & 3) / 2;           // logical chunk
    const int sub = (trj & 1) * 8;                              // byte half within the chunk
    const int r_lo = 4 * half + tre, r_hi = r_lo + 8;
    v_off[0][dt] = r_lo * ROWB + ((lq ^ swz<D>(r_lo)) * 16) + sub;
    v_off[1][dt] = r_hi * ROWB + ((lq ^ swz<D>(r_hi)) * 16) + sub;
  }

  // The wave's rows are positions wp0 .. wp1 of the tile (none when wp1 < wp0).  A key tile wholly
  // after the newest key they see, or (sliding window) wholly before the oldest, changes none of
  // them: on tiles crossing the diagonal the waves whose rows all come before the tile skip it.
  const int wp0 = (32 * w) / G;
  const int wp1 = min((32 * w + 31) / G, n_pos - 1);
  const int wave_newest = ctx + q_off + wp1;
  const int wave_oldest = ctx + q_off + wp0 - a.window + 1;

  // one key tile: S^T, mask, online softmax, O^T += V^T P^T, reading (kl, vl)
  auto tile_math = [&](int kt, const char* kl, const char* vl) {
    if (wp1 < wp0 || kt * kTileKeys > wave_newest || kt * kTileKeys + kTileKeys - 1 < wave_oldest) return;
    // ---- S^T = K Q^T : two 32-key sub-tiles, chains interleaved, operands read one step ahead ----
    floatx16 S0 = mref16, S1 = mref16;                 // -m_ref
    // K operands are read PD k-steps ahead of their products; the scheduling barriers keep the
    // compiler from sinking the reads next to their use (it otherwise waits on every pair)
    constexpr int PD = 2;
    bf16x8 ka[NKK], kb[NKK];
#pragma unroll
    for (int kk = 0; kk < PD; ++kk) {
      ka[kk] = *reinterpret_cast<const bf16x8*>(kl + k_off[kk]);
      kb[kk] = *reinterpret_cast<const bf16x8*>(kl + k_off[kk] + 32 * ROWB);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + PD < NKK) {
        ka[kk + PD] = *reinterpret_cast<const bf16x8*>(kl + k_off[kk + PD]);
        kb[kk + PD] = *reinterpret_cast<const bf16x8*>(kl + k_off[kk + PD] + 32 * ROWB);
      }
      __builtin_amdgcn_sched_barrier(0);
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qreg[kk], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[kk], qreg[kk], S1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- causal mask (only on tiles that cross the diagonal of the first row) and window mask
    //      (only on tiles that start below the last row's oldest visible key) ----
    if (kt * kTileKeys + kTileKeys - 1 > first_pos || kt * kTileKeys < low_edge) {
      const int oldest = pos - a.window + 1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kt * kTileKeys + 8 * (v >> 2) + 4 * half + (v & 3);
        if (key > pos || key < oldest) S0[v] = -INFINITY;
        if (key + 32 > pos || key + 32 < oldest) S1[v] = -INFINITY;
      }
    }

    // ---- online softmax on s - m_ref; the reference moves (O and l rescaled) only when a row has
    //      none yet and sees a key, or its max exceeds the reference by more than 2^8 ----
    float tm = fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) tm = fmaxf(fmaxf(tm, S0[v]), S1[v]);   // one v_max3 per v
    tm = xor32_max(tm);
    const bool need = has_ref ? (tm > 8.f) : (tm > -INFINITY);
    if (__any(need)) {
      float shift = 0.f;                               // new reference - old, this row
      if (need) {
        const float m_new = (float)(__bf16)(m_ref + tm);
        shift = m_new - m_ref;
        const float alpha = has_ref ? fast_exp2(-shift) : 0.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) O[dt][v] *= alpha;
        m_ref = m_new;
        has_ref = true;
#pragma unroll
        for (int v = 0; v < 16; ++v) mref16[v] = -m_new;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) { S0[v] -= shift; S1[v] -= shift; }
    }
    bf16x8 P[4];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      P[v >> 3][v & 7] = (__bf16)fast_exp2(S0[v]);
      P[2 + (v >> 3)][v & 7] = (__bf16)fast_exp2(S1[v]);
    }
    // row sum of the bf16 probabilities the products use, two per v_dot2c_f32_bf16 against (1, 1)
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(P[i], P[i], 0, 1), one2, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(P[i], P[i], 2, 3), one2, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(P[i], P[i], 4, 5), one2, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(P[i], P[i], 6, 7), one2, ps1, false);
    }
    l_run += ps0 + ps1;

    // ---- O^T += V^T P^T : A operand = two 4-key transpose reads per 16-key step ----
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x4 lo[NDT], hi[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        lo[dt] = lds_read_tr(reinterpret_cast<const uint16_t*>(vl + v_off[0][dt] + 16 * kk * ROWB));
        hi[dt] = lds_read_tr(reinterpret_cast<const uint16_t*>(vl + v_off[1][dt] + 16 * kk * ROWB));
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 vop = __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, P[kk], O[dt], 0, 0, 0);
      }
    }
  };

  if constexpr (!KV8) {
    // one LDS variable per buffer and tensor: the compiler then knows that loads landing in one
    // buffer never alias reads of the other, and does not wait for them before those reads
    __shared__ __align__(16) char sK0[TILEB];
    __shared__ __align__(16) char sV0[TILEB];
    __shared__ __align__(16) char sK1[TILEB];
    __shared__ __align__(16) char sV1[TILEB];
    // ---- staging: the wave copies key rows 16bw..16bw+15 of its tensor's tile (one cache block) ----
    // load i of the block covers rows RPI*i .. RPI*i + RPI - 1; lane -> (row lane / CPR, physical
    // chunk lane % CPR), which holds logical chunk (lane % CPR) ^ swz(row).
    uint32_t lane_off[IPB];                         // byte offset within the block, per load
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int rr = RPI * i + lane / CPR;          // row within the block
      const int q = (lane % CPR) ^ swz<D>(16 * bw + rr);
      lane_off[i] = (uint32_t)(rr * rs * 2) + q * 16;
    }
    auto stage = [&](int kt, char* kdst, char* vdst) {
      char* dl = (is_v ? vdst : kdst) + 16 * bw * ROWB;
      const int blk = 4 * kt + bw;
      if ((blk + 1) * kBlock <= sl && blk * kBlock >= lo_req) {   // whole block valid: one table entry
        const char* tb = tbase + (int64_t)win.get(table, bw, 4, n_full, kt) * (kBlock * rs * 2);
        const uint32_t l = __builtin_amdgcn_readfirstlane(lds_u32(dl));
#pragma unroll
        for (int i = 0; i < IPB; ++i) dma16(tb, lane_off[i], l + 1024 * i);
      } else {                                      // edge block: clamp rows into [lo_req, sl)
        const uint32_t l = __builtin_amdgcn_readfirstlane(lds_u32(dl));
#pragma unroll
        for (int i = 0; i < IPB; ++i) {
          const int rr = RPI * i + lane / CPR;
          const int j = min(max(blk * kBlock + rr, lo_req), sl - 1);
          const int q = (lane % CPR) ^ swz<D>(16 * bw + rr);
          const int64_t off = (((int64_t)load_i32_sync(table + (j >> 4)) * kBlock + (j & 15)) * rs) * 2 + q * 16;
          dma16_addr(tbase + off, l + 1024 * i);
        }
      }
    };

    stage(kt_lo, sK0, sV0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // two tiles per iteration so that each buffer is a fixed LDS variable (the second one
    // conditional rather than a break out of the loop: a break leaves the loop-carried values
    // undefined on its path, and the compiler then fills them from a register the last product
    // writes, which makes the wave wait for that product before the barrier)
    for (int kt = kt_lo; kt < n_kt; kt += 2) {
      if (kt + 1 < n_kt) stage(kt + 1, sK1, sV1);     // in flight during this tile's math
      tile_math(kt, sK0, sV0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 1 < n_kt) {
        if (kt + 2 < n_kt) stage(kt + 2, sK0, sV0);
        tile_math(kt + 1, sK1, sV1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    }


  } else {
    constexpr int CPR8 = D / 16;                  // 16-byte chunks per int8 row
    constexpr int RPI8 = 1024 / D;                // int8 rows per wave-wide 1 KiB load
    constexpr int IPB8 = kBlock / RPI8;
    constexpr int TILE8 = kTileKeys * D;          // bytes per staged int8 tile
    __shared__ __align__(16) char sK0[TILEB];      // bf16 tiles the math reads, double buffered
    __shared__ __align__(16) char sV0[TILEB];
    __shared__ __align__(16) char sK1[TILEB];
    __shared__ __align__(16) char sV1[TILEB];
    __shared__ __align__(16) char sK8a[TILE8];     // int8 staging, double buffered
    __shared__ __align__(16) char sV8a[TILE8];
    __shared__ __align__(16) char sK8b[TILE8];
    __shared__ __align__(16) char sV8b[TILE8];
    // staging: plain row-major int8 rows; load i of the wave's block covers rows RPI8*i + lane/CPR8
    uint32_t lane_off8[IPB8];
#pragma unroll
    for (int i = 0; i < IPB8; ++i) {
      const int rr = RPI8 * i + lane / CPR8;
      lane_off8[i] = (uint32_t)(rr * rs) + (lane % CPR8) * 16;
    }
    auto stage8 = [&](int kt, char* kdst, char* vdst) {
      char* dl = (is_v ? vdst : kdst) + 16 * bw * D;
      const int blk = 4 * kt + bw;
      if ((blk + 1) * kBlock <= sl && blk * kBlock >= lo_req) {
        const char* tb = tbase + (int64_t)win.get(table, bw, 4, n_full, kt) * (kBlock * rs);
#pragma unroll
        for (int i = 0; i < IPB8; ++i)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tb + lane_off8[i]),
                                           (__attribute__((address_space(3))) void*)(dl + 1024 * i), 16, 0, 0);
      } else {                                    // edge block: clamp rows into [lo_req, sl)
#pragma unroll
        for (int i = 0; i < IPB8; ++i) {
          const int rr = RPI8 * i + lane / CPR8;
          const int j = min(max(blk * kBlock + rr, lo_req), sl - 1);
          const int64_t off = ((int64_t)table[j >> 4] * kBlock + (j & 15)) * rs + (lane % CPR8) * 16;
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tbase + off),
                                           (__attribute__((address_space(3))) void*)(dl + 1024 * i), 16, 0, 0);
        }
      }
    };
    // conversion: threads 0-255 widen K, 256-511 V (whole waves each); thread -> (row, 16-code
    // piece cj of it), the PPR threads of a row adjacent, so 16 lanes read 256 contiguous bytes.
    // Each piece becomes two bf16 chunks, stored in the order set by the row's parity: the 16
    // stores of a lane group then land on 16 different physical chunks (rows r and r + 1 write
    // chunks of opposite parity under the swizzle), which keeps the stores free of bank conflicts.
    constexpr int PPR = D / 16;                   // 16-code pieces per row
    constexpr int RPP = 256 / PPR;                // rows per pass
    const int ct = tid & 255, cj = ct % PPR, crow0 = ct / PPR;
    const int h0 = crow0 & 1;                     // RPP is even: every pass keeps the parity
    auto widen8 = [](uint32_t w0, uint32_t w1) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(float)(signed char)((e < 4 ? w0 : w1) >> (8 * (e & 3)));
      return o;
    };
    auto convert = [&](const char* k8, const char* v8, char* kd, char* vd) {
      const char* src = is_v ? v8 : k8;
      char* const cdst = is_v ? vd : kd;
#pragma unroll
      for (int u = 0; u < 64 / RPP; ++u) {
        const int crow = crow0 + RPP * u;
        const uint4 x = *reinterpret_cast<const uint4*>(src + crow * D + 16 * cj);
        const bf16x8 first = widen8(h0 ? x.z : x.x, h0 ? x.w : x.y);     // logical chunk 2cj + h0
        const bf16x8 second = widen8(h0 ? x.x : x.z, h0 ? x.y : x.w);    // logical chunk 2cj + 1 - h0
        char* const rowp = cdst + crow * ROWB;
        *reinterpret_cast<bf16x8*>(rowp + (((2 * cj + h0) ^ swz<D>(crow)) * 16)) = first;
        *reinterpret_cast<bf16x8*>(rowp + (((2 * cj + (h0 ^ 1)) ^ swz<D>(crow)) * 16)) = second;
      }
    };

    // Tile kt+1 is widened in the same phase as tile kt's math (other buffers), so one barrier
    // per tile separates the phases: before it, tile kt+1's codes have landed (staged a phase
    // earlier) and tile kt+2's copies are in flight.
    stage8(kt_lo, sK8a, sV8a);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    convert(sK8a, sV8a, sK0, sV0);
    if (kt_lo + 1 < n_kt) stage8(kt_lo + 1, sK8b, sV8b);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kt = kt_lo; kt < n_kt; kt += 2) {
      // tile kt widened in (sK0, sV0); tile kt + 1's codes in b
      if (kt + 1 < n_kt) convert(sK8b, sV8b, sK1, sV1);
      if (kt + 2 < n_kt) stage8(kt + 2, sK8a, sV8a);       // a was widened a phase ago
      tile_math(kt, sK0, sV0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 1 < n_kt) {                                  // (conditional, not a break: see above)
        if (kt + 2 < n_kt) convert(sK8a, sV8a, sK0, sV0);   // tile kt's math is done
        if (kt + 3 < n_kt) stage8(kt + 3, sK8b, sV8b);
        tile_math(kt + 1, sK1, sV1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    }
  }

  // ---- epilogue: O / l, round to bf16, store (lane holds 4 consecutive d per group) ----
  const float lt = xor32_sum(l_run);
  const float inv = 1.f / lt;
  if (row_ok) {
    char* op = reinterpret_cast<char*>(a.out) + ((t * a.num_q_heads + h) * D) * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int dd = 32 * dt + 8 * grp + 4 * half;
        float4 sc = make_float4(inv, inv, inv, inv);
        if constexpr (KV8) {                       // v_scale of channels dd .. dd + 3
          const float4 vs = *reinterpret_cast<const float4*>(a.v_scale + (int64_t)g * D + dd);
          sc = make_float4(inv * vs.x, inv * vs.y, inv * vs.z, inv * vs.w);
        }
        uint2 pk;
        pk.x = pack_bf16x2(O[dt][4 * grp + 0] * sc.x, O[dt][4 * grp + 1] * sc.y);
        pk.y = pack_bf16x2(O[dt][4 * grp + 2] * sc.z, O[dt][4 * grp + 3] * sc.w);
        *reinterpret_cast<uint2*>(op + dd * 2) = pk;
      }
  }
}

hipError_t launch_prefill_tile(const TileArgs& a, int head_dim, bool kv8, hipStream_t s) {
  const int64_t grid = (int64_t)a.num_slots * a.num_kv_heads;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), blk(512);
  if (head_dim == 128) {
    if (kv8) prefill_tile_kernel<128, true><<<g, blk, 0, s>>>(a);
    else prefill_tile_kernel<128, false><<<g, blk, 0, s>>>(a);
  } else if (head_dim == 64) {
    if (kv8) prefill_tile_kernel<64, true><<<g, blk, 0, s>>>(a);
    else prefill_tile_kernel<64, false><<<g, blk, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
