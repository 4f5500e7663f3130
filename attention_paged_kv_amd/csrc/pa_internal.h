// pa_internal.h -- host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Requests with q_len <= kVerifyMax over a bf16 or int8 cache (decode, and a few tokens to
// verify) and every query row of an fp32 batch run on the split-KV decode kernels; longer requests
// over a bf16 or int8 cache run on the MFMA tile kernel.
constexpr int kDefaultSplitTokens = 256;   // keys per decode split (multiple of 16, at most 1024)
constexpr int kI8SplitTokens = 320;        // the same over an 8-bit cache
constexpr int kLongSplitTokens = 384;      // either, when a row may span more than 8192 keys
constexpr int kTileRows = 256;             // query rows (position x head-in-group) per prefill workgroup
constexpr int kMaxTileGroup = 128;         // query heads per KV head the prefill tiles accept
constexpr int kTileKeys = 64;              // keys per MFMA K/V tile
constexpr int kNoWindow = 1 << 30;         // window value meaning "every earlier key"
constexpr int kVerifyMax = 8;              // bf16 requests with q_len <= this run on the split-KV pass

struct AppendArgs {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int64_t num_tokens;
  int64_t row_bytes;      // Hkv * d * esz of the input rows
  const float* k_scale;   // int8 caches: [Hkv][d] scales (row elements share the row index)
  const float* v_scale;   //   nullptr: plain copy
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* out;
  float* part_o;          // [rows][qmax][max_splits][Hq][d]   unnormalised partial outputs
  float* part_ml;         // [rows][qmax][max_splits][Hq][2]   (running max in log2 units, sum)
  int num_seqs;
  int num_rows;           // row slots: requests (bf16, int8) or tokens (fp32)
  int per_token;          // 1: row slot = token index; 0: row slot = request with q_len <= qmax
  int qmax;               // positions a request row may carry (1 for per-token rows)
  int num_q_heads;
  int num_kv_heads;
  int group;              // Hq / Hkv
  int heads_per_wg;       // columns per workgroup: (position, query head) pairs of one KV head
  int max_blocks;
  int split;              // keys per split (stream mode: fewest keys per run)
  int max_splits;         // partial slots per (row, position, head): splits, or pieces in stream mode
  int stream_wgs;         // > 0: stream mode with this many workgroups per head group; 0: splits
  int pair_wgs;           // bf16 split mode: 1 = workgroups of two KV heads, one wave per SIMD; 0 = four
  int window;             // keys a row sees, its own included (kNoWindow: all earlier keys)
  float scale_log2;       // scale * log2(e)
  const float* k_scale;   // int8 caches: [Hkv][d]
  const float* v_scale;
};

struct TileArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* out;
  int num_seqs;
  int min_q;              // requests with q_len >= min_q run here (shorter ones on the decode pass)
  int num_slots;          // upper bound on tiles launched per KV head
  int num_q_heads;
  int num_kv_heads;
  int group;
  int pos_per_tile;       // kTileRows / group
  int max_blocks;
  int window;             // as in DecodeArgs
  float scale_log2;
  const float* k_scale;   // int8 caches: [Hkv][d]
  const float* v_scale;
};

struct CheckArgs {
  const int32_t* slot_mapping;   // append check (nullptr for attention)
  int num_tokens;
  int64_t num_slots;
  const int32_t* block_tables;   // attention check (nullptr for append)
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs;
  int max_blocks;
  int num_blocks;
  int num_q_tokens;
  int window;                    // table entries before the first row's window are not checked
  int max_q_len;                 // > 0: every q_len must be at most this
  int* result;                   // [4]: flag, code, index, value (device, zeroed by caller)
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_decode_split_i8(const DecodeArgs& a, int head_dim, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_prefill_tile(const TileArgs& a, int head_dim, bool kv8, hipStream_t s);
hipError_t launch_check(const CheckArgs& a, hipStream_t s);

}  // namespace pa
