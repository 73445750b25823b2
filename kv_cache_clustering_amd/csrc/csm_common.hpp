// Device pieces shared by the CSM round kernels: row tiles, segment packing, the MFMA
// similarity tile, ordered row copies and flag waits.
#pragma once

#include "device_common.hpp"

namespace csmkv {

template <typename T, int NT = 256, int D = 128, int CMAX = kMaxChunk>
struct Tile {
  static constexpr int ROWB = D * (int)sizeof(T);         // bytes per row (head dim D)
  static constexpr int SEGS = ROWB / 16;                  // 16-byte segments per row
  static constexpr int RPI = NT / SEGS;                   // rows covered by one block-wide load
  static constexpr int NLD = CMAX / RPI;                  // loads per thread for CMAX rows
  static constexpr int EPS = 16 / (int)sizeof(T);         // elements per segment
};

// Sum of squares of one 16-byte segment (fp32; bf16 squares are exact in fp32).
__device__ __forceinline__ float seg_sumsq(u32x4 v, __bf16 *) {
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float lo = bf_lo(v[q]), hi = bf_hi(v[q]);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}
__device__ __forceinline__ float seg_sumsq(u32x4 v, _Float16 *) {
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // fp16 squares are exact in fp32
    const uint32_t w = v[q];
    const float lo = f16_lo(w), hi = f16_hi(w);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}
__device__ __forceinline__ float seg_sumsq(u32x4 v, float *) {
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = __uint_as_float(v[q]);
    s = fmaf(x, x, s);
  }
  return s;
}

// Unpack a segment to fp32 / pack fp32 back to the storage type.
__device__ __forceinline__ void seg_unpack(u32x4 v, float *o, __bf16 *) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = bf_lo(v[q]);
    o[2 * q + 1] = bf_hi(v[q]);
  }
}
__device__ __forceinline__ void seg_unpack(u32x4 v, float *o, _Float16 *) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = v[q];
    o[2 * q] = f16_lo(w);
    o[2 * q + 1] = f16_hi(w);
  }
}
__device__ __forceinline__ void seg_unpack(u32x4 v, float *o, float *) {
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = __uint_as_float(v[q]);
}
__device__ __forceinline__ u32x4 seg_pack(const float *o, __bf16 *) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // v_cvt_pk_bf16_f32: round to nearest even
    const bf16x2 h = {(__bf16)o[2 * q], (__bf16)o[2 * q + 1]};
    v[q] = __builtin_bit_cast(uint32_t, h);
  }
  return v;
}
__device__ __forceinline__ u32x4 seg_pack(const float *o, _Float16 *) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // v_cvt_f16_f32: round to nearest even
    const f16x2 h = {(_Float16)o[2 * q], (_Float16)o[2 * q + 1]};
    v[q] = __builtin_bit_cast(uint32_t, h);
  }
  return v;
}
__device__ __forceinline__ u32x4 seg_pack(const float *o, float *) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(o[q]);
  return v;
}

// S^T tiles for one wave: acc[i][q] = <key of B row ((tl0 + i)*32 + row_q), key of A row a>
// for NTL consecutive 32-row B tiles starting at tl0.
template <int NTL, int D>
__device__ __forceinline__ void sim_tile(const char *tile, int a, int col, int h, f32x16 *acc,
                                         __bf16 *, int tl0 = 0) {
  constexpr int ROWB = Tile<__bf16, 256, D>::ROWB;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int seg = 2 * kk + h;
    u32x4 braw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(2 * a, seg, ROWB));
    bf16x8 bop = __builtin_bit_cast(bf16x8, braw);
#pragma unroll
    for (int tl = 0; tl < NTL; ++tl) {
      const int brow = 2 * ((tl0 + tl) * 32 + col) + 1;
      u32x4 araw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(brow, seg, ROWB));
      bf16x8 aop = __builtin_bit_cast(bf16x8, araw);
      acc[tl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc[tl], 0, 0, 0);
    }
  }
}
template <int NTL, int D>
__device__ __forceinline__ void sim_tile(const char *tile, int a, int col, int h, f32x16 *acc,
                                         _Float16 *, int tl0 = 0) {
  constexpr int ROWB = Tile<_Float16, 256, D>::ROWB;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int seg = 2 * kk + h;
    u32x4 braw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(2 * a, seg, ROWB));
    f16x8 bop = __builtin_bit_cast(f16x8, braw);
#pragma unroll
    for (int tl = 0; tl < NTL; ++tl) {
      const int brow = 2 * ((tl0 + tl) * 32 + col) + 1;
      u32x4 araw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(brow, seg, ROWB));
      f16x8 aop = __builtin_bit_cast(f16x8, araw);
      acc[tl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, acc[tl], 0, 0, 0);
    }
  }
}
template <int NTL, int D>
__device__ __forceinline__ void sim_tile(const char *tile, int a, int col, int h, f32x16 *acc,
                                         float *, int tl0 = 0) {
  constexpr int ROWB = Tile<float, 256, D>::ROWB;
  // Half-wave h supplies elements 8q + 4h + i at k-step 4q + i: every element is used
  // once and both operands use the same assignment.
#pragma unroll 2
  for (int q = 0; q < D / 8; ++q) {
    const int seg = 2 * q + h;
    u32x4 braw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(2 * a, seg, ROWB));
#pragma unroll
    for (int tl = 0; tl < NTL; ++tl) {
      const int brow = 2 * ((tl0 + tl) * 32 + col) + 1;
      u32x4 araw = *reinterpret_cast<const u32x4 *>(tile + lds_swz(brow, seg, ROWB));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(araw[i]),
                                                       __uint_as_float(braw[i]), acc[tl], 0, 0, 0);
    }
  }
}

// Copy `nrows` rows (K, V, N) from src to dst in ascending blocks of ROWS rows.  Each block
// is fully read before any of it is written, so dst <= src (a shift to lower rows) is safe
// in place.
template <typename T, int NT, int D, int ROWS = kMaxChunk>
__device__ void copy_rows(const char *Ks, const char *Vs, const int32_t *Ns, char *Kd, char *Vd,
                          int32_t *Nd, int nrows) {
  using TL = Tile<T, NT, D>;
  constexpr int NB = ROWS / TL::RPI;  // loads per thread per block of ROWS rows
  const int t = threadIdx.x, sg = t % TL::SEGS, r0 = t / TL::SEGS;
  for (int blk = 0; blk < nrows; blk += ROWS) {
    const int nb = min(ROWS, nrows - blk);
    u32x4 kb[NB], vb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = r0 + TL::RPI * i;
      if (r < nb) {
        kb[i] = ld16(Ks + (int64_t)(blk + r) * TL::ROWB + sg * 16);
        vb[i] = ld16(Vs + (int64_t)(blk + r) * TL::ROWB + sg * 16);
      }
    }
    int32_t nv = (t < ROWS && t < nb) ? Ns[blk + t] : 0;
    wait_vm_loads();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = r0 + TL::RPI * i;
      if (r < nb) {
        st16(Kd + (int64_t)(blk + r) * TL::ROWB + sg * 16, kb[i]);
        st16(Vd + (int64_t)(blk + r) * TL::ROWB + sg * 16, vb[i]);
      }
    }
    if (t < ROWS && t < nb) Nd[blk + t] = nv;
    __syncthreads();
  }
}

// Waits until *f is set by another workgroup; false if it is not set within kFlagPolls polls
// (about a second, against the microseconds a wait takes), so that a wait that cannot end turns
// into a reported error instead of a hung launch.
constexpr uint32_t kFlagPolls = 1u << 24;
__device__ __forceinline__ bool wait_flag(const int32_t *f) {
  for (uint32_t i = 0; i < kFlagPolls; ++i) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

}  // namespace csmkv
