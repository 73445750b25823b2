// One Chunked Soft Matching round on the host's CPU cores: the CPU-offloaded clustering variant.
//
// CentroidKV page, 它做不到的事（局限性） → 仍留在 GPU 上 and 技术摘要 → 作者注明的局限性: the
// grouping runs on the GPU, and running it on the CPU and sending only its result to the GPU is
// named as the unexplored alternative.  This file computes the same round as csm_compress
// (Chelsea review, section 三, 分块软匹配算法 steps 1-4; CentroidKV page, 分块软匹配 (CSM) and 聚合)
// over a cache held in host memory; csm_upload_rows (csmkv_abi.cpp) then copies the compacted rows
// to the device cache asynchronously.
//
// Work split: one slice at a time per worker thread (slices taken from a shared counter); inside
// a slice the chunks run in order, each copied to thread-local buffers before its output is
// written, so the in-place compaction (output row base n1 + j (c - m) <= the chunk's first row)
// never overwrites rows that are still to be read.  Per chunk:
//   keys to fp32 (bf16 and fp16 convert exactly), norms and reciprocal norms in fp32;
//   every A x B dot product in fp32 by the widest vector unit the CPU reports at run time
//   (AVX-512, AVX2 + FMA, or scalar), cosine = (dot * 1/|b|) * 1/|a|, the lowest B index on ties;
//   the A edges ordered by a unique 64-bit key (score descending, A index ascending) and the
//   first m = floor(r L / 2) merged: (N_b x_b + sum N_a x_a) / W accumulated in fp32 in ascending
//   A order, rounded to the storage type to nearest, ties to even;
//   kept rows written in their original order.
// Host code only: it shares nothing with the device kernels.
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "csmkv.h"

namespace {

// ------------------------------------------------------------------ storage formats
inline float bits_to_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint32_t f32_to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

inline float bf16_to_f32(uint16_t b) { return bits_to_f32(uint32_t(b) << 16); }

// fp32 -> bfloat16, round to nearest, ties to even (NaN -> quiet NaN)
inline uint16_t f32_to_bf16(float x) {
  uint32_t u = f32_to_bits(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// IEEE binary16 -> fp32 (exact)
inline float f16_to_f32(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16, e = (h >> 10) & 0x1f, m = h & 0x3ffu;
  if (e == 0) {  // zero or subnormal: m * 2^-24
    const float v = std::ldexp(float(m), -24);
    return (h & 0x8000u) ? -v : v;
  }
  if (e == 31) return bits_to_f32(sign | 0x7f800000u | (m << 13));  // inf / NaN
  return bits_to_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

// fp32 -> IEEE binary16, round to nearest, ties to even; overflow to infinity
inline uint16_t f32_to_f16(float x) {
  const uint32_t u = f32_to_bits(x), sign = (u >> 16) & 0x8000u, ax = u & 0x7fffffffu;
  if (ax > 0x7f800000u) return uint16_t(sign | 0x7e00u);           // NaN
  if (ax >= 0x477ff000u) return uint16_t(sign | 0x7c00u);          // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                          // below 2^-14: subnormal
    const float v = bits_to_f32(ax) * 16777216.0f;                 // units of 2^-24, exact
    return uint16_t(sign | uint32_t(std::nearbyint(v)));           // nearest, ties to even
  }
  uint32_t h = ((((ax >> 23) - 127 + 15) & 0x1fu) << 10) | ((ax >> 13) & 0x3ffu);
  const uint32_t rest = ax & 0x1fffu;
  if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) ++h;       // carries into the exponent
  return uint16_t(sign | h);
}

// One row of the storage type <-> fp32.
inline void row_to_f32(const char *src, int dtype, int d, float *dst) {
  if (dtype == CSMKV_F32) {
    std::memcpy(dst, src, size_t(d) * 4);
  } else {
    const uint16_t *s = reinterpret_cast<const uint16_t *>(src);
    if (dtype == CSMKV_BF16)
      for (int k = 0; k < d; ++k) dst[k] = bf16_to_f32(s[k]);
    else
      for (int k = 0; k < d; ++k) dst[k] = f16_to_f32(s[k]);
  }
}
inline void f32_to_row(const float *src, int dtype, int d, char *dst) {
  if (dtype == CSMKV_F32) {
    std::memcpy(dst, src, size_t(d) * 4);
  } else {
    uint16_t *o = reinterpret_cast<uint16_t *>(dst);
    if (dtype == CSMKV_BF16)
      for (int k = 0; k < d; ++k) o[k] = f32_to_bf16(src[k]);
    else
      for (int k = 0; k < d; ++k) o[k] = f32_to_f16(src[k]);
  }
}

// ------------------------------------------------------------------ dot products
// S[i * ld + j] = <A_i, B_j> for fp32 rows of length d, A row-major [nA][d], B given transposed
// (Bt[k * ld + j] = B_j[k], columns nB .. ld - 1 zero; ld a multiple of 32).  Every product is
// summed over k in ascending order with one fused multiply-add per step, so all three forms give
// the same bits.
using DotsFn = void (*)(const float *, const float *, int, int, int, int, float *);

void dots_scalar(const float *A, const float *Bt, int nA, int nB, int ld, int d, float *S) {
  for (int i = 0; i < nA; ++i)
    for (int j = 0; j < nB; ++j) {
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = std::fma(A[size_t(i) * d + k], Bt[size_t(k) * ld + j], acc);
      S[size_t(i) * ld + j] = acc;
    }
}

__attribute__((target("avx2,fma"))) inline float hsum256(__m256 v) {
  __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  s = _mm_add_ps(s, _mm_movehl_ps(s, s));
  s = _mm_add_ss(s, _mm_movehdup_ps(s));
  return _mm_cvtss_f32(s);
}

// Register tiles of R A rows x 16 B columns (AVX2: two 8-wide vectors per column block; AVX-512:
// one 16-wide): each step over k broadcasts R A elements and loads one row of Bt.
template <int R>
__attribute__((target("avx2,fma"))) inline void tile_avx2(const float *A, const float *Bt, int ld,
                                                          int d, int j, float *S) {
  __m256 c[R][2];
  for (int r = 0; r < R; ++r) c[r][0] = c[r][1] = _mm256_setzero_ps();
  for (int k = 0; k < d; ++k) {
    const __m256 b0 = _mm256_loadu_ps(Bt + size_t(k) * ld + j);
    const __m256 b1 = _mm256_loadu_ps(Bt + size_t(k) * ld + j + 8);
    for (int r = 0; r < R; ++r) {
      const __m256 a = _mm256_broadcast_ss(A + size_t(r) * d + k);
      c[r][0] = _mm256_fmadd_ps(a, b0, c[r][0]);
      c[r][1] = _mm256_fmadd_ps(a, b1, c[r][1]);
    }
  }
  for (int r = 0; r < R; ++r) {
    _mm256_storeu_ps(S + size_t(r) * ld + j, c[r][0]);
    _mm256_storeu_ps(S + size_t(r) * ld + j + 8, c[r][1]);
  }
}

__attribute__((target("avx2,fma"))) void dots_avx2(const float *A, const float *Bt, int nA, int nB,
                                                   int ld, int d, float *S) {
  for (int j = 0; j < nB; j += 16) {
    int i = 0;
    for (; i + 6 <= nA; i += 6) tile_avx2<6>(A + size_t(i) * d, Bt, ld, d, j, S + size_t(i) * ld);
    for (; i < nA; ++i) tile_avx2<1>(A + size_t(i) * d, Bt, ld, d, j, S + size_t(i) * ld);
  }
}

template <int R>
__attribute__((target("avx512f"))) inline void tile_avx512(const float *A, const float *Bt, int ld,
                                                           int d, int j, float *S) {
  __m512 c[R][2];
  for (int r = 0; r < R; ++r) c[r][0] = c[r][1] = _mm512_setzero_ps();
  for (int k = 0; k < d; ++k) {
    const __m512 b0 = _mm512_loadu_ps(Bt + size_t(k) * ld + j);
    const __m512 b1 = _mm512_loadu_ps(Bt + size_t(k) * ld + j + 16);
    for (int r = 0; r < R; ++r) {
      const __m512 a = _mm512_set1_ps(A[size_t(r) * d + k]);
      c[r][0] = _mm512_fmadd_ps(a, b0, c[r][0]);
      c[r][1] = _mm512_fmadd_ps(a, b1, c[r][1]);
    }
  }
  for (int r = 0; r < R; ++r) {
    _mm512_storeu_ps(S + size_t(r) * ld + j, c[r][0]);
    _mm512_storeu_ps(S + size_t(r) * ld + j + 16, c[r][1]);
  }
}

__attribute__((target("avx512f"))) void dots_avx512(const float *A, const float *Bt, int nA, int nB,
                                                    int ld, int d, float *S) {
  for (int j = 0; j < nB; j += 32) {  // 32 B columns per tile (ld covers the padding)
    int i = 0;
    for (; i + 12 <= nA; i += 12) tile_avx512<12>(A + size_t(i) * d, Bt, ld, d, j, S + size_t(i) * ld);
    for (; i + 4 <= nA; i += 4) tile_avx512<4>(A + size_t(i) * d, Bt, ld, d, j, S + size_t(i) * ld);
    for (; i < nA; ++i) tile_avx512<1>(A + size_t(i) * d, Bt, ld, d, j, S + size_t(i) * ld);
  }
}

// Reciprocal norms 1 / max(|x|, 1e-12) of n rows (sum of squares in fp32).
using NormsFn = void (*)(const float *, int, int, float *);
// First b in [0, nB) with the largest (dots[b] * rb[b]) * ra (strict >, so the lowest b on
// ties); returns b and the score.
using BestFn = int (*)(const float *, const float *, float, int, float *);
// a[e] = fma(w, x[e], a[e]) for e < d.
using AxpyFn = void (*)(float, const float *, float *, int);

void norms_scalar(const float *rows, int n, int d, float *inv) {
  for (int i = 0; i < n; ++i) {
    float ss = 0.f;
    for (int k = 0; k < d; ++k) ss = std::fma(rows[size_t(i) * d + k], rows[size_t(i) * d + k], ss);
    inv[i] = 1.0f / std::max(std::sqrt(ss), 1e-12f);
  }
}
int best_scalar(const float *dots, const float *rb, float ra, int nB, float *score) {
  float bs = -INFINITY;
  int bi = 0;
  for (int b = 0; b < nB; ++b) {
    const float scv = (dots[b] * rb[b]) * ra;
    if (scv > bs) {
      bs = scv;
      bi = b;
    }
  }
  *score = bs;
  return bi;
}
void axpy_scalar(float w, const float *x, float *a, int d) {
  for (int e = 0; e < d; ++e) a[e] = std::fma(w, x[e], a[e]);
}

__attribute__((target("avx2,fma"))) void norms_avx2(const float *rows, int n, int d, float *inv) {
  for (int i = 0; i < n; ++i) {
    const float *x = rows + size_t(i) * d;
    __m256 c0 = _mm256_setzero_ps(), c1 = c0;
    for (int k = 0; k < d; k += 16) {
      const __m256 a = _mm256_loadu_ps(x + k), b = _mm256_loadu_ps(x + k + 8);
      c0 = _mm256_fmadd_ps(a, a, c0);
      c1 = _mm256_fmadd_ps(b, b, c1);
    }
    inv[i] = 1.0f / std::max(std::sqrt(hsum256(_mm256_add_ps(c0, c1))), 1e-12f);
  }
}
__attribute__((target("avx2,fma"))) int best_avx2(const float *dots, const float *rb, float ra,
                                                  int nB, float *score) {
  const __m256 vra = _mm256_set1_ps(ra), step = _mm256_set1_ps(8.f);
  __m256 vbest = _mm256_set1_ps(-INFINITY), vidx = _mm256_setzero_ps();
  __m256 lane = _mm256_setr_ps(0.f, 1.f, 2.f, 3.f, 4.f, 5.f, 6.f, 7.f);
  int b = 0;
  for (; b + 8 <= nB; b += 8) {  // per lane: the first index of its largest score
    const __m256 sc = _mm256_mul_ps(_mm256_mul_ps(_mm256_loadu_ps(dots + b), _mm256_loadu_ps(rb + b)), vra);
    const __m256 gt = _mm256_cmp_ps(sc, vbest, _CMP_GT_OQ);
    vbest = _mm256_blendv_ps(vbest, sc, gt);
    vidx = _mm256_blendv_ps(vidx, lane, gt);
    lane = _mm256_add_ps(lane, step);
  }
  alignas(32) float bv[8], bi[8];
  _mm256_store_ps(bv, vbest);
  _mm256_store_ps(bi, vidx);
  float bs = -INFINITY;
  int best = 0;
  for (int q = 0; q < 8; ++q)  // across lanes: the largest score, the lowest index on ties
    if (bv[q] > bs || (bv[q] == bs && bv[q] != -INFINITY && int(bi[q]) < best)) {
      bs = bv[q];
      best = int(bi[q]);
    }
  for (; b < nB; ++b) {  // the tail, in order after every earlier index
    const float scv = (dots[b] * rb[b]) * ra;
    if (scv > bs) {
      bs = scv;
      best = b;
    }
  }
  *score = bs;
  return best;
}
__attribute__((target("avx2,fma"))) void axpy_avx2(float w, const float *x, float *a, int d) {
  const __m256 vw = _mm256_set1_ps(w);
  for (int e = 0; e < d; e += 8)
    _mm256_storeu_ps(a + e, _mm256_fmadd_ps(vw, _mm256_loadu_ps(x + e), _mm256_loadu_ps(a + e)));
}

__attribute__((target("avx512f"))) void norms_avx512(const float *rows, int n, int d, float *inv) {
  for (int i = 0; i < n; ++i) {
    const float *x = rows + size_t(i) * d;
    __m512 c = _mm512_setzero_ps();
    for (int k = 0; k < d; k += 16) {
      const __m512 a = _mm512_loadu_ps(x + k);
      c = _mm512_fmadd_ps(a, a, c);
    }
    inv[i] = 1.0f / std::max(std::sqrt(_mm512_reduce_add_ps(c)), 1e-12f);
  }
}
__attribute__((target("avx512f"))) int best_avx512(const float *dots, const float *rb, float ra,
                                                   int nB, float *score) {
  const __m512 vra = _mm512_set1_ps(ra);
  __m512 vbest = _mm512_set1_ps(-INFINITY);
  __m512i vidx = _mm512_setzero_si512();
  __m512i lane = _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  const __m512i step = _mm512_set1_epi32(16);
  int b = 0;
  for (; b + 16 <= nB; b += 16) {  // per lane: the first index of its largest score
    const __m512 sc = _mm512_mul_ps(_mm512_mul_ps(_mm512_loadu_ps(dots + b), _mm512_loadu_ps(rb + b)), vra);
    const __mmask16 gt = _mm512_cmp_ps_mask(sc, vbest, _CMP_GT_OQ);
    vbest = _mm512_mask_mov_ps(vbest, gt, sc);
    vidx = _mm512_mask_mov_epi32(vidx, gt, lane);
    lane = _mm512_add_epi32(lane, step);
  }
  alignas(64) float bv[16];
  alignas(64) int32_t bi[16];
  _mm512_store_ps(bv, vbest);
  _mm512_store_si512(bi, vidx);
  float bs = -INFINITY;
  int best = 0;
  for (int q = 0; q < 16; ++q)  // across lanes: the largest score, the lowest index on ties
    if (bv[q] > bs || (bv[q] == bs && bv[q] != -INFINITY && bi[q] < best)) {
      bs = bv[q];
      best = bi[q];
    }
  for (; b < nB; ++b) {  // the tail, in order after every earlier index
    const float scv = (dots[b] * rb[b]) * ra;
    if (scv > bs) {
      bs = scv;
      best = b;
    }
  }
  *score = bs;
  return best;
}
__attribute__((target("avx512f"))) void axpy_avx512(float w, const float *x, float *a, int d) {
  const __m512 vw = _mm512_set1_ps(w);
  for (int e = 0; e < d; e += 16)
    _mm512_storeu_ps(a + e, _mm512_fmadd_ps(vw, _mm512_loadu_ps(x + e), _mm512_loadu_ps(a + e)));
}

struct Isa {
  DotsFn dots;
  NormsFn norms;
  BestFn best;
  AxpyFn axpy;
  int code;  // CSMKV_HOST_ISA_*
};

Isa pick_isa() {
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx512f"))
    return {dots_avx512, norms_avx512, best_avx512, axpy_avx512, CSMKV_HOST_ISA_AVX512};
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
    return {dots_avx2, norms_avx2, best_avx2, axpy_avx2, CSMKV_HOST_ISA_AVX2};
  return {dots_scalar, norms_scalar, best_scalar, axpy_scalar, CSMKV_HOST_ISA_SCALAR};
}

// ------------------------------------------------------------------ one round
// Merges of a chunk of length L: floor(r L / 2 + 1e-9) in fp64, within [0, ceil(L / 2)].
int merges(double r, int L) {
  if (L < 2) return 0;
  const int m = int(std::floor(r * double(L) * 0.5 + 1e-9));
  return std::max(0, std::min(m, (L + 1) / 2));
}

// Unique key ordering A edges by descending score, then ascending index (-0 folded into +0).
inline uint64_t edge_key(float score, int a) {
  const uint32_t u = f32_to_bits(score + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(ord) << 16) | uint64_t(0xffff - a);
}

struct Params {
  char *K, *V;
  int32_t *N, *lens;
  int64_t S, cap;
  int d, dtype, rowb, n1, n2, c, W;
  double r;
  const uint8_t *mask;
  int32_t *tap_best;
  uint8_t *tap_sel;
  int32_t *tap_src;
  int64_t units;
  Isa isa;
};

// Row stride of the transposed B rows and of the products: nB rounded up to 32 columns.
inline int ld_of(int nB) { return (nB + 31) / 32 * 32; }

struct Scratch {  // per worker thread
  std::vector<char> k, v;
  std::vector<int32_t> n;
  std::vector<float> af, bf, bt, ra, rb, dots, acc, tmp, sc;
  std::vector<int> best, src_list, src_cnt, src_off, outrow;
  std::vector<uint64_t> keys;
  std::vector<uint8_t> sel;
  explicit Scratch(const Params &p) {
    const size_t c = size_t(p.c), d = size_t(p.d), na = (c + 1) / 2;
    k.resize(c * p.rowb);
    v.resize(c * p.rowb);
    n.resize(c);
    af.resize(na * d);
    bf.resize(na * d);
    bt.resize(d * ld_of(na));
    ra.resize(na);
    rb.resize(na);
    dots.resize(na * ld_of(na));
    acc.resize(2 * d);
    tmp.resize(d);
    sc.resize(na);
    best.resize(na);
    src_list.resize(na);
    src_cnt.resize(na);
    src_off.resize(na + 1);
    outrow.resize(c);
    keys.resize(na);
    sel.resize(na);
  }
};

void round_slice(const Params &p, int64_t z, Scratch &w) {
  const int s = p.lens[z];
  const int n1 = p.n1, n2 = p.n2, c = p.c, d = p.d, rowb = p.rowb;
  char *Kz = p.K + z * p.cap * rowb;
  char *Vz = p.V + z * p.cap * rowb;
  int32_t *Nz = p.N + z * p.cap;
  int32_t *src = p.tap_src ? p.tap_src + z * p.cap : nullptr;
  const int M = s - n1 - n2;
  if (M < 2) {
    if (src)
      for (int i = 0; i < s; ++i) src[i] = i;
    return;
  }
  const int nch = (M + c - 1) / c;
  int out = n1;  // next output row
  for (int j = 0; j < nch; ++j) {
    const int start = n1 + j * c, L = std::min(c, M - j * c);
    const int m = merges(p.r, L), nA = (L + 1) / 2, nB = L / 2;
    // the chunk's rows to local buffers (the output may overlap them)
    std::memcpy(w.k.data(), Kz + int64_t(start) * rowb, size_t(L) * rowb);
    std::memcpy(w.v.data(), Vz + int64_t(start) * rowb, size_t(L) * rowb);
    std::memcpy(w.n.data(), Nz + start, size_t(L) * 4);
    std::fill(w.sel.begin(), w.sel.begin() + nA, uint8_t(0));
    std::fill(w.src_cnt.begin(), w.src_cnt.begin() + std::max(nB, 1), 0);
    for (int i = 0; i < nA; ++i) w.best[i] = -1;
    if (nB > 0) {
      for (int i = 0; i < nA; ++i) row_to_f32(w.k.data() + size_t(2 * i) * rowb, p.dtype, d, &w.af[size_t(i) * d]);
      for (int i = 0; i < nB; ++i) row_to_f32(w.k.data() + size_t(2 * i + 1) * rowb, p.dtype, d, &w.bf[size_t(i) * d]);
      p.isa.norms(w.af.data(), nA, d, w.ra.data());
      p.isa.norms(w.bf.data(), nB, d, w.rb.data());
      const int ld = ld_of(nB);
      for (int k = 0; k < d; ++k) {  // B transposed, padding columns zero
        float *col = &w.bt[size_t(k) * ld];
        for (int b = 0; b < nB; ++b) col[b] = w.bf[size_t(b) * d + k];
        for (int b = nB; b < ld; ++b) col[b] = 0.f;
      }
      p.isa.dots(w.af.data(), w.bt.data(), nA, nB, ld, d, w.dots.data());
      for (int i = 0; i < nA; ++i) {  // best B: ascending, strict >, so the lowest wins a tie
        float bs;
        const int bi = p.isa.best(&w.dots[size_t(i) * ld], w.rb.data(), w.ra[i], nB, &bs);
        w.best[i] = bi;
        w.sc[i] = bs;
        w.keys[i] = edge_key(bs, i);
      }
      if (m > 0) {  // the m largest keys
        std::vector<uint64_t> &k = w.keys;
        std::nth_element(k.begin(), k.begin() + (m - 1), k.begin() + nA, std::greater<uint64_t>());
        for (int q = 0; q < m; ++q) w.sel[0xffff - int(k[q] & 0xffffu)] = 1;
      }
    }
    // sources of every target in ascending A order
    for (int i = 0; i < nA; ++i)
      if (w.sel[i]) ++w.src_cnt[w.best[i]];
    w.src_off[0] = 0;
    for (int b = 0; b < nB; ++b) w.src_off[b + 1] = w.src_off[b] + w.src_cnt[b];
    for (int b = 0; b < nB; ++b) w.src_cnt[b] = 0;
    for (int i = 0; i < nA; ++i)
      if (w.sel[i]) {
        const int b = w.best[i];
        w.src_list[w.src_off[b] + w.src_cnt[b]++] = i;
      }
    // kept rows in order (from row n1 + j (c - m) on); merge targets averaged
    for (int t = 0; t < L; ++t) {
      if (!(t & 1) && w.sel[t >> 1]) continue;
      const int64_t o = out++;
      char *kd = Kz + o * rowb, *vd = Vz + o * rowb;
      const int b = t >> 1;
      if ((t & 1) && w.src_cnt[b] > 0) {
        int64_t W = w.n[t];
        for (int q = w.src_off[b]; q < w.src_off[b + 1]; ++q) W += w.n[2 * w.src_list[q]];
        for (int pass = 0; pass < 2; ++pass) {
          const char *rows = pass == 0 ? w.k.data() : w.v.data();
          float *a = w.acc.data();
          row_to_f32(rows + size_t(t) * rowb, p.dtype, d, w.tmp.data());
          const float nb = float(w.n[t]);
          for (int e = 0; e < d; ++e) a[e] = nb * w.tmp[e];
          for (int q = w.src_off[b]; q < w.src_off[b + 1]; ++q) {
            const int ar = 2 * w.src_list[q];
            row_to_f32(rows + size_t(ar) * rowb, p.dtype, d, w.tmp.data());
            const float na = float(w.n[ar]);
            p.isa.axpy(na, w.tmp.data(), a, d);
          }
          const float Wf = float(W);
          for (int e = 0; e < d; ++e) a[e] = a[e] / Wf;
          f32_to_row(a, p.dtype, d, pass == 0 ? kd : vd);
        }
        Nz[o] = int32_t(W);
      } else {
        std::memcpy(kd, w.k.data() + size_t(t) * rowb, rowb);
        std::memcpy(vd, w.v.data() + size_t(t) * rowb, rowb);
        Nz[o] = w.n[t];
      }
      if (src) src[o] = start + t;
    }
    if (p.tap_best) {
      const int64_t o = (z * p.units + j) * p.W;
      for (int i = 0; i < p.W; ++i) {
        p.tap_best[o + i] = i < nA && nB > 0 ? w.best[i] : -1;
        p.tap_sel[o + i] = i < nA ? w.sel[i] : 0;
      }
    }
  }
  // the recent rows follow the last chunk's output
  const int64_t so = s - n2;
  std::memmove(Kz + int64_t(out) * rowb, Kz + so * rowb, size_t(n2) * rowb);
  std::memmove(Vz + int64_t(out) * rowb, Vz + so * rowb, size_t(n2) * rowb);
  std::memmove(Nz + out, Nz + so, size_t(n2) * 4);
  if (src) {
    for (int i = 0; i < n1; ++i) src[i] = i;
    for (int i = 0; i < n2; ++i) src[out + i] = int32_t(so + i);
  }
  p.lens[z] = out + n2;
}

}  // namespace

extern "C" {

int csm_host_isa(void) { return pick_isa().code; }

int csm_compress_host(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                      int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                      int32_t num_threads, int32_t *best_b, uint8_t *selected, int32_t *src_pos) {
  if (cache == nullptr) return CSMKV_EINVAL;
  if (cache->dtype != CSMKV_BF16 && cache->dtype != CSMKV_F32 && cache->dtype != CSMKV_F16)
    return CSMKV_EDTYPE;
  if (cache->num_slices < 0 || cache->cap < 1) return CSMKV_EINVAL;
  if (cache->d != 64 && cache->d != 128) return CSMKV_EUNSUPPORTED;
  if (cache->cap > (int64_t(1) << 24)) return CSMKV_EUNSUPPORTED;
  if (n1 < 0 || n2 < 0 || c < 2 || !(r >= 0.0 && r <= 1.0)) return CSMKV_EINVAL;
  if (c > 512) return CSMKV_EUNSUPPORTED;
  if (num_threads < 0) return CSMKV_EINVAL;
  if ((best_b == nullptr) != (selected == nullptr)) return CSMKV_EINVAL;
  if (cache->num_slices == 0) return CSMKV_OK;
  if (!K || !V || !N || !lens) return CSMKV_EINVAL;
  for (int64_t z = 0; z < cache->num_slices; ++z)  // every length checked before anything changes
    if (lens[z] < 0 || int64_t(lens[z]) > cache->cap) return CSMKV_EINVAL;
  Params p;
  p.K = static_cast<char *>(K);
  p.V = static_cast<char *>(V);
  p.N = N;
  p.lens = lens;
  p.S = cache->num_slices;
  p.cap = cache->cap;
  p.d = cache->d;
  p.dtype = cache->dtype;
  p.rowb = cache->d * (cache->dtype == CSMKV_F32 ? 4 : 2);
  p.n1 = n1;
  p.n2 = n2;
  p.c = c;
  p.W = c <= 256 ? 128 : 256;
  p.r = r;
  p.mask = outlier_mask;
  p.tap_best = best_b;
  p.tap_sel = selected;
  p.tap_src = src_pos;
  const int64_t Mmax = int64_t(cache->max_len) - n1 - n2;
  p.units = (Mmax >= 2 ? (Mmax + c - 1) / c : 0) + 1;  // the device round's tap layout
  p.isa = pick_isa();
  if (best_b) {
    int64_t need = 0;  // every slice's chunks must fit the tap layout of max_len
    for (int64_t z = 0; z < p.S; ++z)
      if (!(outlier_mask && outlier_mask[z])) {
        const int64_t M = int64_t(lens[z]) - n1 - n2;
        need = std::max<int64_t>(need, M >= 2 ? (M + c - 1) / c : 0);
      }
    if (need + 1 > p.units) return CSMKV_EINVAL;
  }
  int threads = num_threads > 0 ? num_threads : int(std::max(1u, std::thread::hardware_concurrency()));
  threads = int(std::min<int64_t>(threads, p.S));
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    Scratch w(p);
    for (int64_t z = next++; z < p.S; z = next++)
      if (!(outlier_mask && outlier_mask[z])) round_slice(p, z, w);
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < threads; ++i) pool.emplace_back(worker);
  worker();
  for (auto &t : pool) t.join();
  return CSMKV_OK;
}

}  // extern "C"
