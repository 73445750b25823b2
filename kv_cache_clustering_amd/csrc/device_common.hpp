// Device helpers shared by the libcsmkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csmkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxChunk = 256;       // chunk capacity of the main kernels (128 x 128 tile)
constexpr int kMaxChunkWide = 512;   // capacity of the wide-chunk kernels (256 x 256 tile)
constexpr int kDeviceError = -6;     // CSMKV_EDEVICE

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// bf16 pair packed in one dword -> fp32 (exact)
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp16 pair packed in one dword -> fp32 (exact)
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16 bits, round to nearest, ties to even (NaN -> quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Byte offset of 16-byte segment `seg` of row `row` in an LDS tile with `rowbytes` per row.
// The XOR spreads the rows a half-wave reads at one segment (consecutive A or B rows,
// i.e. rows 2i or 2i+1) over distinct bank groups; it stays inside the row (at most 16
// segments are permuted).
__device__ __forceinline__ int lds_swz(int row, int seg, int rowbytes) {
  const int mask = (rowbytes / 16 - 1) & 15;
  return row * rowbytes + ((seg ^ ((row >> 1) & mask)) << 4);
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}
// Sum over aligned groups of LANES (8, 16 or 32) lanes; every lane of a group receives it.
template <int LANES>
__device__ __forceinline__ float lanes_sum(float x) {
  static_assert(LANES == 8 || LANES == 16 || LANES == 32, "8, 16 or 32 lanes");
  x += dpp_f<0xb1>(x);
  x += dpp_f<0x4e>(x);
  x += dpp_f<0x141>(x);                    // now summed over 8 lanes
  if (LANES >= 16) x += dpp_f<0x140>(x);  // 16
  if (LANES == 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ void wait_vm_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Orders this wave's LDS accesses before and after it for the compiler (acquire-release fence at
// wavefront scope: no instruction and no wait is emitted, since a wave's LDS operations execute in
// program order, but no load or store is moved across it).  Used where lanes of one wave read what
// other lanes of it wrote.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

constexpr int kBufWord3 = 0x00020000;  // raw (unformatted) buffer, 32-bit data format
// A pointer that holds the same value in every lane, moved to scalar registers (the compiler
// cannot always prove that a slice index found at run time is wave-uniform).
__device__ __forceinline__ void *wave_uniform(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<void *>(lo | (hi << 32));
}

// Exclusive prefix sum of one value per thread over a block of NT threads; *total gets the
// block's sum.  wsum: NT / 64 ints of LDS.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int *total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    before += i < w ? wsum[i] : 0;
    all += wsum[i];
  }
  *total = all;
  return before + incl - v;
}

// Merge count of a chunk of length L: floor(r * L / 2 + 1e-9) in fp64 (no contraction),
// clamped to [0, ceil(L/2)]; 0 for L < 2.
__device__ __forceinline__ int merge_count_dev(double r, int L) {
  if (L < 2) return 0;
  double x = __dadd_rn(__dmul_rn(__dmul_rn(r, (double)L), 0.5), 1e-9);
  int m = (int)floor(x);
  int hi = (L + 1) / 2;
  return m < 0 ? 0 : (m > hi ? hi : m);
}

}  // namespace csmkv
