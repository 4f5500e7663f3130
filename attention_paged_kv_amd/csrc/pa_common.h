// pa_common.h -- device helpers shared by the libpa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;       // tokens per cache block
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// bf16 <-> fp32.  Widening is exact; narrowing uses the hardware round-to-nearest-even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;           // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;           // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // lane i <-> 7-i within each 8-lane half row
constexpr int kDppMirror = 0x140;        // lane i <-> 15-i within each 16-lane row

// Sum over aligned groups of N lanes (N in {8, 16, 32}); every lane of a group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine lane l with lane l ^ 32 (v_permlane32_swap: returns {x[l], x[l ^ 32]} in some order).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Combine lane l with lane l ^ 16 (v_permlane16_swap).
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Block ids a wave will visit, 64 at a time: lane i holds the id of the wave's i-th block of the
// current window, so the loop takes each id with one v_readlane instead of a memory round trip.
struct BlockWindow {
  int ids = 0;
  int base = -(1 << 30);
  // ids of blocks first + stride * (base + lane), for base + lane < count
  __device__ __forceinline__ void load(const int32_t* table, int first, int stride, int count, int new_base) {
    base = new_base;
    const int i = new_base + (int)(threadIdx.x & 63);
    ids = i < count ? table[first + stride * i] : 0;
  }
  // id of the wave's k-th block (k < count)
  __device__ __forceinline__ int get(const int32_t* table, int first, int stride, int count, int k) {
    if (k - base >= 64 || k < base) load(table, first, stride, count, k);
    return __builtin_amdgcn_readlane(ids, k - base);
  }
};

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, input lane 4e + c gives
// the address of 4 consecutive elements of row e, columns 4c..4c+3 of a 4 x 16 tile; output lane
// j receives column j of the tile: rows 0..3.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(const __attribute__((address_space(3))) uint16_t*)p);
}

// 16 bytes per lane from global memory straight into LDS: lane i writes lds + 16 i, reading
// gbase + voff (gbase uniform across the wave, voff per lane).  Issued as inline assembly so the
// compiler does not see the copy: it keeps counting its own loads precisely instead of waiting for
// every outstanding copy before each LDS read.  The caller waits for completion itself
// (s_waitcnt vmcnt) before the data is read.  M0 is saved and restored around the copy.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  const uint64_t gb = (uint64_t)(uintptr_t)gbase;          // the address operand must be scalar
  gbase = (const void*)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(gb >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gb));
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(voff), "s"(gbase), "s"(lds) : "memory");
}

// As dma16, with a per-lane 64-bit global address.
__device__ __forceinline__ void dma16_addr(const void* gaddr, uint32_t lds) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(gaddr), "s"(lds) : "memory");
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa
