// Log-degree decode attention O = Softmax(q K^T / sqrt(d) + log N) V over a clustered
// cache with grouped-query heads (Chelsea review, section 三, 核心公式: attention with
// cluster degrees n_t; Algorithm 1 decode output), and the Algorithm 1 append step.
//
// Split-K over the sequence, HBM-bound:
//   dec_prep    : (calls over more than 1024 slices) one workgroup validates lens[], gives
//                 every slice ceil(len / tsplit) work items and scans them into item offsets.
//                 tsplit (512 to 2048 tokens) is chosen on the host from the slice count and
//                 the length bound so that a call has about 2048 items.  Smaller calls plan
//                 in the split kernel itself, from the total length (a wave-level scan for up
//                 to 64 slices, an LDS scan beyond): about one item per CU for a layer's few
//                 slices, items of up to 2048 tokens for many slices.
//   dec_split   : workgroups stride over the work items (at most 2048 workgroups).  A work
//                 item is up to tsplit tokens of one slice, shared by the G query heads of
//                 that KV head, so K, V and N are read from HBM once per step.  Each wave
//                 streams a quarter of the item: 16 B per lane per row, 16-token sub-blocks
//                 with the next two sub-blocks' loads in flight while the current one is
//                 computed; base-2 online softmax (log2 N added, log2 e folded into the
//                 scale).  bf16 / fp16: q.k and P.V on MFMA tiles (described below); fp32:
//                 FMAs with a DPP reduction over the lanes of a row, and at G = 8 two
//                 workgroups of four heads each.  Waves merge in LDS; each item writes one
//                 (max, sum, 0, 0, o[d]) partial per head.
//   dec_combine : one 1024-thread workgroup per slice (per (slice, head), 256 threads, for
//                 calls over at most 64 slices) merges the item partials by log-sum-exp (a
//                 running maximum per thread over item groups in parallel, then the groups
//                 merged against their common maximum); for kv_append_decode_attn_logn it also
//                 merges the appended token as one more partial and writes it into the cache.
#include <algorithm>
#include <mutex>

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace csmkv {

// Scratch memory of the allocation-free decode entry point: what a caller's workspace holds
// for decode_attn_logn (item offsets, item table, per-item partials), in one fixed array.
// Each GPU the library runs on holds its own copy until the process ends; host code reaches
// it only through the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kTSplitMin = 512, kTSplitMax = 2048;  // tokens per work item
constexpr int64_t kItemTarget = 2048;               // work items a call aims for
// floats per (item, head) partial: (max, sum, 0, 0, o[d]), 16-byte aligned rows
template <int D>
constexpr int part_width() { return 4 + D; }
constexpr int kDecThreads = 256;
constexpr int kCombThreads = 1024;  // dec_combine workgroup
#ifndef DEC_NS
#define DEC_NS 3
#endif
// Split workgroups per call at most (eight per CU); larger calls loop over their items.
constexpr int64_t kMaxSplitGroups = 256 * 8;
// Calls over at most kInlineSlices slices skip the plan kernel: every split workgroup scans
// the lengths into LDS itself, picks the item size from the total length and finds its items
// there.  Larger calls keep the plan kernel (its table costs no LDS per slice).
constexpr int kInlineSlices = 1024;
constexpr int kInlineTSplitMin = 256, kInlineItems = 256;  // one item per CU

static bool dec_inline(int64_t num_slices, int32_t) { return num_slices <= kInlineSlices; }

// Upper bound on the items of an in-kernel plan.  The item size ts is at least 256 tokens,
// and at least T / 256 unless it is capped at kTSplitMax, so the item count
// sum ceil(s_z / ts) < T / ts + S is below S + 256, or S + T / kTSplitMax when capped.
static int64_t dec_inline_items(int64_t num_slices, int32_t max_len) {
  const int64_t by_min = num_slices * (int64_t)((max_len + kInlineTSplitMin - 1) / kInlineTSplitMin);
  const int64_t capped = (num_slices * (int64_t)max_len + kTSplitMax - 1) / kTSplitMax;
  return std::min(by_min, num_slices + std::max<int64_t>(kInlineItems, capped));
}

// Item size of an in-kernel plan from the total length T of the call: about one item per CU
// (a short call is bound by each wave's chain of dependent loads, so it pays to spread it over
// every CU once), a multiple of 16 tokens, within [kInlineTSplitMin, kTSplitMax].
__device__ __forceinline__ int inline_split_tokens(int T) {
  const int ts = ((T + kInlineItems - 1) / kInlineItems + 15) / 16 * 16;
  return min(max(ts, kInlineTSplitMin), kTSplitMax);
}

// First token of item p when a slice of s tokens is cut into cnt items whose lengths differ
// by at most one token (the first s % cnt items take the extra token; cnt = ceil(s / item
// size), so no item is longer than the item size).  32-bit arithmetic only: p * (s / cnt)
// is at most s.
__device__ __forceinline__ int item_bound(int p, int s, int cnt) {
  const int q = s / cnt, rem = s - q * cnt;
  return p * q + min(p, rem);
}

__device__ __forceinline__ bool len_ok(const DecArgs &a, int s) {
  return s >= 0 && s <= a.max_len && (int64_t)s <= a.cap;
}

__global__ void __launch_bounds__(1024) dec_prep(DecArgs a) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x;
  const int64_t S = a.num_slices;
  const int64_t per = (S + 1023) / 1024;
  const int64_t z0 = t * per, z1 = min(S, z0 + per);
  int local = 0;
  for (int64_t z = z0; z < z1; ++z) {
    const int s = a.lens[z];
    const bool ok = len_ok(a, s);
    if (!ok) atomicExch(a.err, kDeviceError);
    local += ok ? (s + a.tsplit - 1) / a.tsplit : 0;
  }
  int total;
  int run = block_excl_scan<1024>(local, wsum, &total);
  for (int64_t z = z0; z < z1; ++z) {
    a.item_off[z] = run;
    const int s = a.lens[z];
    a.s_in[z] = s;  // the length as read, for the combine kernel's fused append
    const int cnt = len_ok(a, s) ? (s + a.tsplit - 1) / a.tsplit : 0;
    for (int p = 0; p < cnt; ++p)  // (slice, first token, end token): one load in dec_split
      *reinterpret_cast<int4 *>(a.item_zp + 4 * (int64_t)(run + p)) =
          make_int4((int)z, item_bound(p, s, cnt), item_bound(p + 1, s, cnt), 0);
    run += cnt;
  }
  if (t == 1023) a.item_off[S] = total;
}

template <typename T, int G, int D>
struct DecTile {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int LPR = ROWB / 16;     // lanes per row
  static constexpr int RPW = 64 / LPR;      // rows per wave-wide load
  static constexpr int NR = G >= 8 ? 2 : 4;  // wave loads per sub-block (fewer for 8 heads a wave)
  static constexpr int NS = DEC_NS;          // register stages
  static constexpr int SUB = NR * RPW;      // rows per sub-block
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane
};

__device__ __forceinline__ float seg_dot(u32x4 k, const u32x4 &q, __bf16 *) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copy the element to a scalar first: a bit_cast of the vector element directly was
    // lowered to the same source register for every i
    const uint32_t kw = k[i], qw = q[i];
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                        __builtin_bit_cast(bf16x2, qw), s, false);
  }
  return s;
}
__device__ __forceinline__ float seg_dot(u32x4 k, const u32x4 &q, _Float16 *) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t kw = k[i], qw = q[i];
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kw), __builtin_bit_cast(f16x2, qw), s,
                               false);
  }
  return s;
}
__device__ __forceinline__ float seg_dot(u32x4 k, const u32x4 &q, float *) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(k[i]), __uint_as_float(q[i]), s);
  return s;
}
__device__ __forceinline__ void seg_to_f32(u32x4 v, float *o, __bf16 *) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = bf_lo(v[i]);
    o[2 * i + 1] = bf_hi(v[i]);
  }
}
__device__ __forceinline__ void seg_to_f32(u32x4 v, float *o, _Float16 *) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    o[2 * i] = f16_lo(w);
    o[2 * i + 1] = f16_hi(w);
  }
}
__device__ __forceinline__ void seg_to_f32(u32x4 v, float *o, float *) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One sub-block of a wave's token range held in registers: NR wave loads of K and V rows
// (16 B per lane per row) and the degrees of the lane's rows.
template <int NR>
struct DecStage {
  u32x4 k[NR], v[NR];
  int32_t n[NR];
};

// A wave's rows [wb, we) of one slice as three buffer resources (K, V, N).  Loads through
// them are range-checked by the hardware: a row at or past `we` reads as zeros without touching
// memory, so every load of the stream is issued unconditionally.  (Loads guarded by per-lane
// branches made the compiler wait for all outstanding loads before each sub-block, which turned
// the register stages into one memory round trip per sub-block.)
struct DecRows {
  __amdgpu_buffer_rsrc_t k, v, n;
};
__device__ __forceinline__ DecRows dec_rows(const char *Kz, const char *Vz, const int32_t *Nz,
                                            int rowb, int wb, int we) {
  const int rows = __builtin_amdgcn_readfirstlane(max(we - wb, 0));
  return {__builtin_amdgcn_make_buffer_rsrc(wave_uniform(Kz + (int64_t)wb * rowb), 0, rows * rowb,
                                            kBufWord3),
          __builtin_amdgcn_make_buffer_rsrc(wave_uniform(Vz + (int64_t)wb * rowb), 0, rows * rowb,
                                            kBufWord3),
          __builtin_amdgcn_make_buffer_rsrc(wave_uniform(Nz + wb), 0, rows * 4, kBufWord3)};
}

// Rows rel .. rel + SUB - 1 (relative to wb) of the wave's range, 16 B per lane per row.
// NTL: non-temporal loads (each row is read by one wave only); plain loads where two waves
// read the same rows, so that the second read is served by the cache.
template <typename T, int G, int D, bool NTL = true>
__device__ __forceinline__ void dec_load(DecStage<DecTile<T, G, D>::NR> &st, const DecRows &rs,
                                         int rel, int rw, int sg) {
  using DT = DecTile<T, G, D>;
  constexpr int aux = NTL ? 2 : 0;  // nt
#pragma unroll
  for (int i = 0; i < DT::NR; ++i) {
    const int row = rel + DT::RPW * i + rw;
    const int off = row * DT::ROWB + sg * 16;
    st.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.k, off, 0, aux));
    st.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.v, off, 0, aux));
    st.n[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs.n, row * 4, 0, 0);
  }
}

// Online-softmax update of (mrun, lrun, o) with one sub-block, base 2.
template <typename T, int G, int D>
__device__ __forceinline__ void dec_compute(const DecStage<DecTile<T, G, D>::NR> &st, int sb, int we, int rw,
                                            const u32x4 *qv, float scale_log2, float *mrun,
                                            float *lrun, float (*o)[DecTile<T, G, D>::EPL]) {
  using DT = DecTile<T, G, D>;
  constexpr int EPL = DT::EPL;
  T *tsel = nullptr;
  const float NEG_INF = -__builtin_inff();
  float zs[DT::NR][G], msf[G];
#pragma unroll
  for (int i = 0; i < DT::NR; ++i) {
    const bool ok = sb + DT::RPW * i + rw < we;
    const float ln = __builtin_amdgcn_logf((float)st.n[i]);  // log2
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float d = lanes_sum<DT::LPR>(seg_dot(st.k[i], qv[h], tsel));
      zs[i][h] = ok ? fmaf(d, scale_log2, ln) : NEG_INF;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = zs[0][h];
#pragma unroll
    for (int i = 1; i < DT::NR; ++i) mx = fmaxf(mx, zs[i][h]);
#pragma unroll
    for (int o2 = DT::LPR; o2 < 64; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
    const float mn = fmaxf(mrun[h], mx);
    // while every row so far has degree 0 the maximum is -inf: exponentiate against 0 instead,
    // which gives such rows weight 0 (as log 0 = -inf does) rather than NaN
    msf[h] = mn == NEG_INF ? 0.f : mn;
    const float alpha = fast_exp2(mrun[h] - msf[h]);
    mrun[h] = mn;
    lrun[h] *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
  }
#pragma unroll
  for (int i = 0; i < DT::NR; ++i) {
    float vf[EPL];
    seg_to_f32(st.v[i], vf, tsel);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = fast_exp2(zs[i][h] - msf[h]);
      lrun[h] += pr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pr, vf[e], o[h][e]);
    }
  }
}

// bf16 and fp16 caches run q.k and P.V on MFMA (16 x 16 tiles, heads padded to 16; fp32 caches
// keep the VALU path above).  A wave takes 16-token sub-blocks; lane l covers token row l mod 16
// and lane group g = l / 16:
//   K and V rows are loaded as whole rows (non-temporal, the VALU path's pattern) and staged in
//   per-wave LDS tiles (rows padded by 8 bytes so both read patterns below hit distinct banks);
//   q.k : v_mfma_f32_16x16x32_bf16 with A = K rows from the tile (lane: row l mod 16, 16 bytes at
//         64 kk + 16 g) and B = q (lane: head l mod 16, the same bytes), D / 32 steps; lane l
//         receives the scores of tokens 4g .. 4g + 3 for head l mod 16;
//   P.V : v_mfma_f32_16x16x16_bf16 with A = P (head l mod 16, tokens 4g .. 4g + 3: the lane's own
//         scores, so P needs no exchange) and B = V (tokens 4g .. 4g + 3, column l mod 16 of a
//         16-column block), read across the V tile's rows.  P enters as two terms of the storage
//         type, p = hi + lo (hi = RNE(p), lo = RNE(p - hi); fp16 on p * 2^14), which keeps it to
//         about 2^-17 (bf16) or 2^-22 (fp16) relative; the sum of P is taken in fp32 from p.
//         Lane l holds O rows (heads) 4g .. 4g + 3, column l mod 16 of each block.
template <typename T>
constexpr bool dec_mfma() { return __is_same(T, __bf16) || __is_same(T, _Float16); }
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
// fp16 P terms carry this factor (an exact power of two, removed from O at the end) so that
// neither term of p = hi + lo falls into fp16's subnormal range for p >= 2^-17
constexpr float kF16PScale = 16384.f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct MfStage {
  static constexpr int NR = D / 32;  // wave loads per 16-row sub-block (512 / D rows each)
  u32x4 k[NR], v[NR];
  int32_t n[4];
};
template <int D>
constexpr int mf_stride() { return 2 * D + 8; }  // LDS bytes per staged row (bank spread)

// Sub-block rows rel .. rel + 15 of the wave's range (relative to its first row).  K and V are
// read as whole rows, 16 bytes per lane, 512 / D rows per wave load, non-temporal (each row is
// read once); lane_kv = (l / (D / 8)) * row bytes + 16 (l mod (D / 8)) is the lane's fixed part
// of the address, and the sub-block's, wave-uniform, goes in the scalar offset, so no address
// register is rewritten in the loop (one that shared registers with an in-flight load made the
// loop wait for every load).  The degrees of the tokens 4g .. 4g + 3 the lane scores come as
// lane_n = 16 g plus 4 i.
template <int D>
__device__ __forceinline__ void mf_load(MfStage<D> &st, const DecRows &rs, int rel, int lane_kv,
                                        int lane_n) {
  constexpr int ROWB = 2 * D, NR = D / 32, RPW = 512 / D;
  const int soff = __builtin_amdgcn_readfirstlane(rel * ROWB);
  const int soff_n = __builtin_amdgcn_readfirstlane(rel * 4);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    st.k[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.k, lane_kv + i * RPW * ROWB, soff, 2));
    st.v[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.v, lane_kv + i * RPW * ROWB, soff, 2));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.n[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs.n, lane_n + 4 * i, soff_n, 0);
}

// Online-softmax update with one sub-block, base 2.  mrun / lrun: head l mod 16 (lrun over the
// lane's tokens only); o[eb]: heads 4g .. 4g + 3 of column block eb.  kt, vt: this wave's LDS
// tiles (16 rows each).
template <typename T, int D>
__device__ __forceinline__ void mf_compute(const MfStage<D> &st, const u32x4 *qop,
                                           float scale_log2, float &mrun, float &lrun,
                                           f32x4 *o, char *kt, char *vt, int l) {
  constexpr int NR = D / 32, KK = D / 32, EB = D / 16, ST = mf_stride<D>(), LPR = D / 8;
  const int g = l >> 4, c = l & 15;
  // the sub-block's K rows into LDS as loaded (row l / LPR + 512 / D * i, segment l mod LPR),
  // 8 bytes at a time (the padded rows are 8-byte aligned).  The staged rows are read by other
  // lanes of the wave: each fence keeps a tile's writes before its reads (and the one at the end
  // keeps this sub-block's reads before the next one's writes); a wave's LDS accesses then
  // execute in that order, so no barrier or wait is needed.
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    uint2 *dk = reinterpret_cast<uint2 *>(kt + (l / LPR + (512 / D) * i) * ST + 16 * (l % LPR));
    dk[0] = make_uint2(st.k[i][0], st.k[i][1]);
    dk[1] = make_uint2(st.k[i][2], st.k[i][3]);
  }
  wave_lds_order();
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint2 *src = reinterpret_cast<const uint2 *>(kt + c * ST + 64 * kk + 16 * g);
    const uint2 lo = src[0], hi = src[1];
    const u32x4 kw = {lo.x, lo.y, hi.x, hi.y};
    if constexpr (__is_same(T, __bf16))
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw),
                                                   __builtin_bit_cast(bf16x8, qop[kk]), sc, 0, 0, 0);
    else
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kw),
                                                  __builtin_bit_cast(f16x8, qop[kk]), sc, 0, 0, 0);
  }
  // the V rows into their tile while the score MFMAs run
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    uint2 *dv = reinterpret_cast<uint2 *>(vt + (l / LPR + (512 / D) * i) * ST + 16 * (l % LPR));
    dv[0] = make_uint2(st.v[i][0], st.v[i][1]);
    dv[1] = make_uint2(st.v[i][2], st.v[i][3]);
  }
  wave_lds_order();
  // scores: a row past the range has N = 0 (range-checked load), so log2 N = -inf drops it
  float z[4], mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = fmaf(sc[i], scale_log2, __builtin_amdgcn_logf((float)st.n[i]));
    mx = fmaxf(mx, z[i]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(mrun, mx);
  // while every row so far has degree 0 the maximum is -inf: exponentiate against 0 instead,
  // which gives such rows weight 0 (as log 0 = -inf does) rather than NaN
  const float msf = mn == -__builtin_inff() ? 0.f : mn;
  const float alpha = fast_exp2(mrun - msf);
  mrun = mn;
  float p[4], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = fast_exp2(z[i] - msf);
    ps += p[i];
  }
  lrun = fmaf(lrun, alpha, ps);
  // rescale factors of the heads this lane's O rows hold (lane h holds head h's factor)
  float al[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
  typedef T tx4 __attribute__((ext_vector_type(4)));
  constexpr float psc = __is_same(T, __bf16) ? 1.f : kF16PScale;
  tx4 ph, pl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ps_i = p[i] * psc;
    ph[i] = (T)ps_i;
    pl[i] = (T)(ps_i - (float)ph[i]);
  }
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    tx4 vop;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vop[j] = *reinterpret_cast<const T *>(vt + (4 * g + j) * ST + 2 * (16 * eb + c));
#pragma unroll
    for (int i = 0; i < 4; ++i) o[eb][i] *= al[i];
    if constexpr (__is_same(T, __bf16)) {
      o[eb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vop, o[eb], 0, 0, 0);
      o[eb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vop, o[eb], 0, 0, 0);
    } else {
      o[eb] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vop, o[eb], 0, 0, 0);
      o[eb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vop, o[eb], 0, 0, 0);
    }
  }
  wave_lds_order();  // every read of this sub-block's tiles before the next one's writes
}

// G = 8 splits the heads into two sets (0-3 and 4-7), each served by its own workgroup, so that
// every wave holds the registers of four heads (eight spill) and a CU still holds two
// workgroups.  Work unit v = 16k + j takes item 8k + (j mod 8) for head set j / 8: the two
// halves of an item run in workgroups whose indices differ by 8, which the dispatcher places
// on the same XCD (workgroups go round-robin over the 8 XCDs), so the second read of a row is
// served by that XCD's L2.
template <typename T, int G>
constexpr int dec_head_sets() { return G >= 8 && !dec_mfma<T>() ? 2 : 1; }
// Work units of a call with `items` items, the item of unit v and its head set.
template <int HS>
__host__ __device__ constexpr int64_t dec_units(int64_t items) {
  return HS == 1 ? items : (items + 7) / 8 * 16;
}
template <int HS>
__device__ __forceinline__ int dec_unit_item(int v) { return HS == 1 ? v : (v >> 4) * 8 + (v & 7); }
template <int HS>
__device__ __forceinline__ int dec_unit_set(int v) { return HS == 1 ? 0 : (v >> 3) & 1; }

// INL: the items are found from the lengths in the kernel (calls over at most kInlineSlices
// slices), else read from the plan kernel's table.
template <typename T, int G, int D, bool INL>
__global__ void __launch_bounds__(kDecThreads, 2) dec_split(DecArgs a) {
  constexpr bool MF = dec_mfma<T>();
  constexpr int HS = dec_head_sets<T, G>(), GW = G / HS, NT = kDecThreads;
  using DT = DecTile<T, GW, D>;
  constexpr int ROWB = DT::ROWB, LPR = DT::LPR, RPW = DT::RPW, SUB = DT::SUB, EPL = DT::EPL;
  constexpr int PW = part_width<D>();  // (max, sum, pad, pad, o[d]) per head
  __shared__ float s_part[4][GW][PW];
  __shared__ __attribute__((aligned(16))) char s_kt[4][MF ? 16 * mf_stride<D>() : 16];
  __shared__ __attribute__((aligned(16))) char s_vt[4][MF ? 16 * mf_stride<D>() : 16];
  __shared__ int32_t s_off[kInlineSlices + 1], s_len[kInlineSlices], s_wsum[NT / 64],
      s_wsum2[NT / 64];
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int sg = l % LPR, rw = l / LPR;
  const int S = (int)a.num_slices;
  const float NEG_INF = -__builtin_inff();
  int total, ts = a.tsplit;
  // Calls over at most 64 slices (a layer's KV heads) plan inside every wave, in registers: lane
  // z holds slice z's length and its inclusive item offset, so neither the plan nor the search
  // for an item's slice needs a barrier or LDS.
  const bool wave_plan = INL && S <= 64;
  int w_len = 0, w_incl = 0;
  if (INL && wave_plan) {
    const int sl = l < S ? a.lens[l] : 0;
    const bool ok = l >= S || len_ok(a, sl);
    w_len = ok ? sl : 0;
    int incl = w_len;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (l >= o) incl += y;
    }
    ts = __builtin_amdgcn_readfirstlane(inline_split_tokens(__builtin_amdgcn_readlane(incl, 63)));
    const int cnt = (w_len + ts - 1) / ts;
    incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (l >= o) incl += y;
    }
    w_incl = incl;
    total = __builtin_amdgcn_readlane(incl, 63);
    if (blockIdx.x == 0 && w == 0) {  // offsets for the combine kernel; a bad length is sticky
      if (l < S) {
        a.item_off[l] = incl - cnt;
        a.s_in[l] = sl;  // the length as read, for the combine kernel's fused append
      }
      if (l == 0) a.item_off[S] = total;
      const uint64_t badm = __ballot(!ok);
      if (l == 0 && badm != 0) atomicExch(a.err, kDeviceError);
    }
  } else if constexpr (INL) {
    // item counts of all slices, scanned into LDS (a bad length counts 0 items).  Workgroup
    // 0 also stores the offsets for the combine kernel and, for a bad length, sets the
    // (sticky) error word.
    const int per = (S + NT - 1) / NT, z0 = t * per, z1 = min(S, z0 + per);
    int sum = 0, bad = 0;
    for (int z = z0; z < z1; ++z) {
      const int s = a.lens[z];
      const bool ok = len_ok(a, s);
      bad |= !ok;
      s_len[z] = ok ? s : 0;
      sum += ok ? s : 0;
    }
    int tot_len;
    block_excl_scan<NT>(sum, s_wsum, &tot_len);
    ts = __builtin_amdgcn_readfirstlane(inline_split_tokens(tot_len));
    int local = 0;
    for (int z = z0; z < z1; ++z) local += (s_len[z] + ts - 1) / ts;
    int run = block_excl_scan<NT>(local, s_wsum2, &total);
    total = __builtin_amdgcn_readfirstlane(total);
    for (int z = z0; z < z1; ++z) {
      s_off[z] = run;
      if (blockIdx.x == 0) {
        a.item_off[z] = run;
        a.s_in[z] = a.lens[z];  // the length as read, for the combine kernel's fused append
      }
      run += (s_len[z] + ts - 1) / ts;
    }
    if (blockIdx.x == 0 && t == 0) a.item_off[S] = total;
    const int any_bad = __syncthreads_or(bad);
    if (blockIdx.x == 0 && t == 0 && any_bad) atomicExch(a.err, kDeviceError);
  } else {
    total = a.item_off[S];
  }
  // one work item: tokens [tok0, tok1) of slice z for the heads of head set hs
  auto process = [&](int item, int hs, int64_t z, int tok0, int tok1) {
    const int64_t g = z / a.H_kv, kvh = z % a.H_kv;
    const char *Kz = a.K + z * a.cap * ROWB;
    const char *Vz = a.V + z * a.cap * ROWB;
    const int32_t *Nz = a.N + z * a.cap;
    const int wq = (tok1 - tok0 + 3) / 4;  // the item's tokens over the four waves
    // the wave's token range, in scalar registers (the buffer resources must be wave-uniform)
    const int wb = __builtin_amdgcn_readfirstlane(tok0 + w * wq);
    const int we = __builtin_amdgcn_readfirstlane(min(tok1, wb + wq));
    const DecRows rs = dec_rows(Kz, Vz, Nz, ROWB, wb, we);
    if constexpr (MF) {
      constexpr int KK = D / 32, EB = D / 16, NS = DEC_NS;
      const int gq = l >> 4, c = l & 15;
      // q of head c as the B operand (zeros for the padding heads c >= G), loaded first
      u32x4 qop[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 qw = {0u, 0u, 0u, 0u};
        if (c < G) qw = ld16(a.q + ((g * a.H_q + kvh * G + c) * (int64_t)D) * 2 + 64 * kk + 16 * gq);
        qop[kk] = qw;
      }
      // each stage's loads are issued as one group, in stage order, ahead of the compute that
      // precedes their use (sched_barrier keeps the scheduler from interleaving or sinking them:
      // loads retire in order, so a reordered stage makes the first sub-block wait for all)
      const int lane_kv = (l / (D / 8)) * ROWB + 16 * (l % (D / 8)), lane_n = 16 * gq;
      MfStage<D> st[NS];
#pragma unroll
      for (int k = 0; k + 1 < NS; ++k) {
        mf_load<D>(st[k], rs, k * 16, lane_kv, lane_n);
        __builtin_amdgcn_sched_barrier(0);
      }
      float mrun = NEG_INF, lrun = 0.f;
      f32x4 o[EB];
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) o[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int sb = wb; sb < we; sb += NS * 16) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const int cur = sb + k * 16;
          if (cur >= we) break;
          mf_load<D>(st[(k + NS - 1) % NS], rs, cur + (NS - 1) * 16 - wb, lane_kv, lane_n);
          __builtin_amdgcn_sched_barrier(0);
          mf_compute<T, D>(st[k], qop, a.scale_log2, mrun, lrun, o, s_kt[w], s_vt[w], l);
        }
      }
      lrun += __shfl_xor(lrun, 16);
      lrun += __shfl_xor(lrun, 32);
      if (l < G) {
        s_part[w][l][0] = mrun;
        s_part[w][l][1] = lrun;
      }
      constexpr float pinv = __is_same(T, __bf16) ? 1.f : 1.f / kF16PScale;
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * gq + i < G) s_part[w][4 * gq + i][4 + 16 * eb + c] = o[eb][i] * pinv;
    } else {
    // this lane's q segment for each head of the wave's head set, loaded first: loads retire in
    // order, so q issued after the stages would make the first sub-block wait for all of them
    u32x4 qv[GW];
#pragma unroll
    for (int h = 0; h < GW; ++h)
      qv[h] = ld16(a.q + ((g * a.H_q + kvh * G + hs * GW + h) * (int64_t)D) * sizeof(T) + sg * 16);
    // NS register stages: the next NS - 1 sub-blocks load while the current one is computed
    constexpr int NS = DT::NS;
    DecStage<DT::NR> st[NS];
#pragma unroll
    for (int k = 0; k + 1 < NS; ++k) dec_load<T, GW, D, HS == 1>(st[k], rs, k * SUB, rw, sg);
    float mrun[GW], lrun[GW], o[GW][EPL];
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      mrun[h] = NEG_INF;
      lrun[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }
    for (int sb = wb; sb < we; sb += NS * SUB) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int cur = sb + k * SUB, nxt = cur + (NS - 1) * SUB;
        if (cur >= we) break;
        // stage (k + NS - 1) % NS was computed last: refill it with the sub-block NS - 1 ahead
        // (past the range the loads read zeros and move no data)
        dec_load<T, GW, D, HS == 1>(st[(k + NS - 1) % NS], rs, nxt - wb, rw, sg);
        dec_compute<T, GW, D>(st[k], cur, we, rw, qv, a.scale_log2, mrun, lrun, o);
      }
    }
    // sum the row groups of the wave (they hold different tokens, same segment)
#pragma unroll
    for (int h = 0; h < GW; ++h) {
#pragma unroll
      for (int o2 = LPR; o2 < 64; o2 <<= 1) lrun[h] += __shfl_xor(lrun[h], o2);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int o2 = LPR; o2 < 64; o2 <<= 1) o[h][e] += __shfl_xor(o[h][e], o2);
    }
    if (rw == 0) {
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        if (sg == 0) {
          s_part[w][h][0] = mrun[h];
          s_part[w][h][1] = lrun[h];
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_part[w][h][4 + sg * EPL + e] = o[h][e];
      }
    }
    }  // VALU path
    __syncthreads();
    // this head set's partials: heads hs * GW .. hs * GW + GW - 1 of the item, contiguous
    float *dst = a.part + ((int64_t)item * G + hs * GW) * PW;
    for (int i = t; i < GW * PW; i += NT) {
      const int h = i / PW, k = i % PW;
      float M = NEG_INF;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_part[ww][h][0]);
      float v = 0.f;
      if (k == 0) {
        v = M;
      } else if (k == 2 || k == 3) {
        v = 0.f;
      } else {
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float mw = s_part[ww][h][0];
          if (mw != NEG_INF) v += fast_exp2(mw - M) * s_part[ww][h][k];
        }
      }
      dst[i] = v;
    }
    __syncthreads();
  };
  if constexpr (INL) {
    // workgroups stride over the items (one each when the grid covers them).  The item's
    // slice is the last z with s_off[z] <= item (slices without items share their offset
    // with the next one).  The LDS values are the same in every lane; readfirstlane keeps
    // the search and the item bounds in scalar registers.
    for (int v = blockIdx.x; v < dec_units<HS>(total); v += gridDim.x) {
      const int item = dec_unit_item<HS>(v), hs = dec_unit_set<HS>(v);
      if (item >= total) continue;
      int z, first, len;
      if (wave_plan) {
        // the item's slice: the number of slices whose items all lie before it
        z = __popcll(__ballot(w_incl <= item));
        len = __builtin_amdgcn_readlane(w_len, z);
        first = __builtin_amdgcn_readlane(w_incl, z) - (len + ts - 1) / ts;
      } else {
        int lo = 0, hi = S - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (__builtin_amdgcn_readfirstlane(s_off[mid]) <= item) lo = mid; else hi = mid - 1;
        }
        z = lo;
        first = __builtin_amdgcn_readfirstlane(s_off[lo]);
        len = __builtin_amdgcn_readfirstlane(s_len[lo]);
      }
      const int p = item - first, cnt = (len + ts - 1) / ts;
      process(item, hs, z, item_bound(p, len, cnt), item_bound(p + 1, len, cnt));
    }
  } else {
    for (int v = blockIdx.x; v < dec_units<HS>(total); v += gridDim.x) {
      const int item = dec_unit_item<HS>(v), hs = dec_unit_set<HS>(v);
      if (item >= total) continue;
      const int4 it4 = *reinterpret_cast<const int4 *>(a.item_zp + 4 * (int64_t)item);
      process(item, hs, it4.x, it4.y, it4.z);
    }
  }
}

// One workgroup per slice, every head at once, in one pass over the partials: each thread
// takes 4 output elements of one head and one of kCombThreads / (D / 4 * G) item groups and sums
// the partials against a running maximum (rescaling its sums when the maximum grows), four
// independent items per step, so a slice of up to 4 items per group needs one round trip to
// memory; the item groups are then merged through LDS against their common maximum and divided.
// One element of the storage type as fp32.
template <typename T>
__device__ __forceinline__ float as_f32(const T *p) {
  if constexpr (__is_same(T, __bf16))
    return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
  else
    return (float)*p;
}

// Threads of a combine workgroup serving HPW of a slice's G heads: 256 for one head (calls over
// few slices spread the merge over G workgroups per slice), kCombThreads for all G.
template <int G, int HPW>
constexpr int comb_threads() { return HPW == 1 && G > 1 ? 256 : kCombThreads; }

template <typename T, int G, int D, int HPW>
__global__ void __launch_bounds__((comb_threads<G, HPW>())) dec_combine(DecArgs a) {
  constexpr int NT = comb_threads<G, HPW>();
  constexpr int PW = part_width<D>();
  constexpr int CPH = D / 4;               // 4-element columns per head
  constexpr int COLS = CPH * HPW;          // columns over the workgroup's heads
  constexpr int IG = NT / COLS;            // item groups
  __shared__ __attribute__((aligned(16))) float s_acc[IG][HPW][D];
  __shared__ float s_l[IG][HPW], s_m[IG][HPW];
  __shared__ float s_zn[HPW];  // fused append: the new token's base-2 logit for each head
  const int64_t z = blockIdx.x / (G / HPW);
  const int hb = (int)(blockIdx.x % (G / HPW)) * HPW;  // the workgroup's first head
  const int t = threadIdx.x;
  const int64_t g = z / a.H_kv, kvh = z % a.H_kv;
  const float NEG_INF = -__builtin_inff();
  const int i0 = a.item_off[z], i1 = a.item_off[z + 1];
  // Fused append: the slice appends the token (if its length is below cap) and attends over the
  // appended length, which must lie within max_len (else the error word is set and the output is
  // zeros, as a separate append and attention would give).  The split kernel covered the rows
  // before the token and recorded the length it read in s_in; the token enters here as one more
  // partial with degree 1.  Loads for it are issued before the partial loop and used after it
  // (so they wait with it): waves 0 .. HPW-1 load q_h and the token's key and form its logits;
  // wave 0 of the slice's first workgroup loads the token's K and V rows (a 16-byte segment per
  // lane) and appends the token to the cache.
  const bool fuse = a.k_new != nullptr;
  auto appends = [&](int s) { return s >= 0 && (int64_t)s < a.cap; };
  auto attends = [&](int s) {
    const int s_att = appends(s) ? s + 1 : s;
    return s_att >= 0 && s_att <= a.max_len && (int64_t)s_att <= a.cap;
  };
  constexpr int RB = D * (int)sizeof(T), SEGR = RB / 16;  // 16-byte segments of a row
  static_assert(2 * SEGR <= 64, "one wave copies the K and V rows");
  static_assert(NT / 64 >= HPW, "a wave per head for the token's logit");
  const int wv = t >> 6, ln = t & 63;
  const int s_old = fuse ? a.s_in[z] : 0;
  const bool appender = fuse && hb == 0 && wv == 0;
  u32x4 seg = {0u, 0u, 0u, 0u};
  float qx[D / 64], kx[D / 64];
  if (fuse) {
    if (appender) {
      if (ln < SEGR)
        seg = ld16(a.k_new + z * RB + ln * 16);
      else if (ln < 2 * SEGR)
        seg = ld16(a.v_new + z * RB + (ln - SEGR) * 16);
    }
    if (wv < HPW) {  // head hb + wv's q and the token's key, elements ln + 64 e
      const T *qh =
          reinterpret_cast<const T *>(a.q) + (g * a.H_q + kvh * G + hb + wv) * (int64_t)D;
      const T *kn = reinterpret_cast<const T *>(a.k_new) + z * D;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) {
        qx[e] = as_f32(qh + ln + 64 * e);
        kx[e] = as_f32(kn + ln + 64 * e);
      }
    }
  }
  // one pass: a running maximum per thread, the sums rescaled when it grows
  const int col = t % COLS, grp = t / COLS, hl = col / CPH, h = hb + hl, e4 = (col % CPH) * 4;
  float M = NEG_INF, acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f, L = 0.f;
  auto rescale = [&](float mnew) {
    if (mnew > M) {
      const float sc = M == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(M - mnew);
      L *= sc;
      acc0 *= sc;
      acc1 *= sc;
      acc2 *= sc;
      acc3 *= sc;
      M = mnew;
    }
  };
  auto add = [&](float m, float lsum, float4 o) {
    const float wgt = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(m - M);
    L = fmaf(wgt, lsum, L);
    acc0 = fmaf(wgt, o.x, acc0);
    acc1 = fmaf(wgt, o.y, acc1);
    acc2 = fmaf(wgt, o.z, acc2);
    acc3 = fmaf(wgt, o.w, acc3);
  };
  int it = i0 + grp;
  for (; it + 3 * IG < i1; it += 4 * IG) {
    float m[4], ls[4];
    float4 o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float *pp = a.part + ((int64_t)(it + k * IG) * G + h) * PW;
      const float4 head = *reinterpret_cast<const float4 *>(pp);
      m[k] = head.x;
      ls[k] = head.y;
      o[k] = *reinterpret_cast<const float4 *>(pp + 4 + e4);
    }
    rescale(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])));
#pragma unroll
    for (int k = 0; k < 4; ++k) add(m[k], ls[k], o[k]);
  }
  for (; it < i1; it += IG) {
    const float *pp = a.part + ((int64_t)it * G + h) * PW;
    const float4 head = *reinterpret_cast<const float4 *>(pp);
    rescale(head.x);
    add(head.x, head.y, *reinterpret_cast<const float4 *>(pp + 4 + e4));
  }
  const bool app = fuse && appends(s_old), att_ok = !fuse || attends(s_old);
  if (fuse) {
    if (wv < HPW) {  // head hb + wv's logit of the token, in fp32 (exact storage-type products)
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) x = fmaf(qx[e], kx[e], x);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
      if (ln == 0) s_zn[wv] = x * a.scale_log2;  // + log2(1)
    }
    if (appender) {  // the token into the cache (nothing in this call reads those rows again)
      if (app) {
        const int64_t row = z * a.cap + s_old;
        if (ln < SEGR)
          st16(a.K_app + row * RB + ln * 16, seg);
        else if (ln < 2 * SEGR)
          st16(a.V_app + row * RB + (ln - SEGR) * 16, seg);
      }
      if (ln == 0) {
        if (app) {
          a.N_app[z * a.cap + s_old] = 1;
          a.lens_app[z] = s_old + 1;
        }
        if (!(app && att_ok)) atomicExch(a.err, kDeviceError);
      }
    }
  }
  // every column of (grp, hl) saw the same maxima, so one of them records M and L
  *reinterpret_cast<float4 *>(&s_acc[grp][hl][e4]) = make_float4(acc0, acc1, acc2, acc3);
  if (e4 == 0) {
    s_l[grp][hl] = L;
    s_m[grp][hl] = M;
  }
  __syncthreads();
  const bool extra = app && att_ok;  // the appended token enters the merge
  for (int i = t; i < HPW * D; i += NT) {
    const int hh = i / D, d = i % D;
    float Mx = NEG_INF;
#pragma unroll
    for (int q = 0; q < IG; ++q) Mx = fmaxf(Mx, s_m[q][hh]);
    const float zn = extra ? s_zn[hh] : NEG_INF;
    Mx = fmaxf(Mx, zn);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int q = 0; q < IG; ++q) {
      const float mq = s_m[q][hh];
      const float wq = mq == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mq - Mx);
      num = fmaf(wq, s_acc[q][hh][d], num);
      den = fmaf(wq, s_l[q][hh], den);
    }
    if (extra) {
      const float wn = __builtin_amdgcn_exp2f(zn - Mx);
      num = fmaf(wn, as_f32(reinterpret_cast<const T *>(a.v_new) + z * D + d), num);
      den += wn;
    }
    a.O[(g * a.H_q + kvh * G + hb + hh) * (int64_t)D + d] =
        (fuse && !att_ok) ? 0.f : den > 0.f ? num / den : 0.f;
  }
}

template <typename T, int D, bool INL>
static int launch_dec_t(const DecArgs &a, int G, int grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((dec_split<T, 1, D, INL>), dim3(grid), dim3(kDecThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((dec_split<T, 2, D, INL>), dim3(grid), dim3(kDecThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((dec_split<T, 4, D, INL>), dim3(grid), dim3(kDecThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((dec_split<T, 8, D, INL>), dim3(grid), dim3(kDecThreads), 0, st, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <typename T, int D>
static int launch_dec_t(const DecArgs &a, int G, int grid, hipStream_t st) {
  return a.inline_items ? launch_dec_t<T, D, true>(a, G, grid, st)
                        : launch_dec_t<T, D, false>(a, G, grid, st);
}

// Calls over at most this many slices (a layer's KV heads) merge with a workgroup per (slice,
// head): G times the workgroups, each reading a quarter of the slice's partials at G = 4, so
// the few slices of a per-layer call are not merged on a handful of CUs.  The result is the same
// bit for bit (each head's merge is unchanged).
constexpr int64_t kCombPerHeadSlices = 64;

template <typename T, int G, int D>
static void launch_combine_g(const DecArgs &a, hipStream_t st) {
  if (G > 1 && a.num_slices <= kCombPerHeadSlices)
    hipLaunchKernelGGL((dec_combine<T, G, D, 1>), dim3((uint32_t)(a.num_slices * G)),
                       dim3(comb_threads<G, 1>()), 0, st, a);
  else
    hipLaunchKernelGGL((dec_combine<T, G, D, G>), dim3((uint32_t)a.num_slices),
                       dim3(comb_threads<G, G>()), 0, st, a);
}

template <typename T, int D>
static int launch_combine_t(const DecArgs &a, int G, hipStream_t st) {
  switch (G) {
    case 1: launch_combine_g<T, 1, D>(a, st); break;
    case 2: launch_combine_g<T, 2, D>(a, st); break;
    case 4: launch_combine_g<T, 4, D>(a, st); break;
    case 8: launch_combine_g<T, 8, D>(a, st); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int D>
static int launch_combine(const DecArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == kDtypeF32 ? launch_combine_t<float, D>(a, G, st)
         : dtype == kDtypeF16 ? launch_combine_t<_Float16, D>(a, G, st)
                              : launch_combine_t<__bf16, D>(a, G, st);
}

template <int D>
static int launch_split(const DecArgs &a, int dtype, int G, int grid, hipStream_t st) {
  return dtype == kDtypeF32   ? launch_dec_t<float, D>(a, G, grid, st)
         : dtype == kDtypeF16 ? launch_dec_t<_Float16, D>(a, G, grid, st)
                              : launch_dec_t<__bf16, D>(a, G, grid, st);
}

int32_t dec_split_tokens(int64_t num_slices, int32_t max_len) {
  const int64_t want = num_slices * (int64_t)max_len / kItemTarget;
  int32_t ts = kTSplitMin;
  while (ts < kTSplitMax && ts < want) ts *= 2;
  return ts;
}

int64_t dec_max_items(int64_t num_slices, int32_t max_len) {
  if (dec_inline(num_slices, max_len)) return dec_inline_items(num_slices, max_len);
  const int32_t ts = dec_split_tokens(num_slices, max_len);
  return num_slices * (int64_t)((max_len + ts - 1) / ts);
}

int noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_decode_table(const DecArgs &args, int dtype, int d, int G, int64_t max_items,
                        hipStream_t st) {
  DecArgs a = args;
  a.inline_items = 0;
  const bool sets2 = G >= 8 && dtype == kDtypeF32;  // dec_head_sets<T, G>() == 2
  const int64_t units = sets2 ? dec_units<2>(max_items) : max_items;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(units, kMaxSplitGroups));
  int rc = d == 64 ? launch_split<64>(a, dtype, G, grid, st) : launch_split<128>(a, dtype, G, grid, st);
  if (rc) return rc;
  return d == 64 ? launch_combine<64>(a, dtype, G, st) : launch_combine<128>(a, dtype, G, st);
}

int launch_decode(const DecArgs &args, int dtype, int d, int G, int64_t max_items, hipStream_t st) {
  DecArgs a = args;
  a.inline_items = dec_inline(a.num_slices, a.max_len);
  if (!a.inline_items) {
    hipLaunchKernelGGL(dec_prep, dim3(1), dim3(1024), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  // G = 8: twice the units, in groups of 16 (kMaxSplitGroups is a multiple of 16, so a
  // workgroup's units keep their partner 8 indices away in every pass)
  const bool sets2 = G >= 8 && dtype == kDtypeF32;  // dec_head_sets<T, G>() == 2
  const int64_t units = sets2 ? dec_units<2>(max_items) : max_items;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(units, kMaxSplitGroups));
  int rc = d == 64 ? launch_split<64>(a, dtype, G, grid, st) : launch_split<128>(a, dtype, G, grid, st);
  if (rc) return rc;
  return d == 64 ? launch_combine<64>(a, dtype, G, st) : launch_combine<128>(a, dtype, G, st);
}

// ------------------------------------------------------------------ append
// K[s] = k, V[s] = v, N[s] = 1, s = s + 1 for every slice (Chelsea review, Algorithm 1
// decode update).  16 lanes of one wave serve one slice (one 16-byte segment each for
// bf16 rows; two for fp32 rows), so the lens read precedes its update in program order.


__global__ void __launch_bounds__(256) kv_append_kernel(AppArgs a) {
  const int64_t z = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sg = threadIdx.x & 15;
  if (z >= a.num_slices) return;
  const int s = a.lens[z];
  const bool ok = s >= 0 && (int64_t)s < a.cap;
  if (ok) {
    for (int off = sg * 16; off < a.rowb; off += 256) {
      st16(a.K + (z * a.cap + s) * a.rowb + off, ld16(a.k_new + z * a.rowb + off));
      st16(a.V + (z * a.cap + s) * a.rowb + off, ld16(a.v_new + z * a.rowb + off));
    }
  }
  if (sg == 0) {
    if (ok) {
      a.N[z * a.cap + s] = 1;
      a.lens[z] = s + 1;
    } else if (a.err != nullptr) {
      atomicExch(a.err, kDeviceError);
    }
  }
}

// Resets an error word to 0 (a kernel rather than a memset node, so that it can be captured in
// a graph and replayed).
__global__ void clear_word_kernel(int32_t *w) { *w = 0; }

int launch_clear(int32_t *word, hipStream_t st) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, word);
  return (int)hipGetLastError();
}

int launch_append(const AppArgs &a, hipStream_t st) {
  const int64_t threads = a.num_slices * 16;
  if (threads == 0) return 0;
  hipLaunchKernelGGL(kv_append_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace csmkv
