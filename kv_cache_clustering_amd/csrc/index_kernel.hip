// Hierarchical centroid index over a clustered cache, and log-N decode attention over the rows
// it keeps.
//
// LycheeCluster page, 方法论 §2 层次 KV 索引: each block's keys summarised by a centroid, the
// centroids arranged in a binary tree whose node distances obey the triangle inequality, and the
// query walking the tree and dropping whole subtrees whose centroid is too far; §3 流式懒更新:
// appends update the newest leaf, upper centroids are refreshed lazily.  Applied to the cache
// Chunked Soft Matching leaves (rows with degrees N; Chelsea review, section 三, 核心公式).
//
// Per slice the index is a ball tree in heap order over P leaf slots (P = 2^ceil(log2(cap / B)),
// fixed by the capacity so that appends always find their leaf): node u holds a centre mu_u
// (fp32, d floats), a radius rho_u, the largest log2 N of its rows and its degree total.  A leaf
// is a block of B consecutive rows: mu = degree-weighted mean of its keys, rho = largest distance
// of a key from mu; an inner node: mu = degree-weighted mean of its children's centres, rho =
// max over children of |mu_c - mu| + rho_c, so each child ball lies inside its parent's.  Radii
// are computed in fp32 and rounded up by a relative 2^-18, which covers the rounding of the
// distance sums, so the balls stay bounding.
//
// For a query q every key k of a ball has q.k <= q.mu + |q| rho, so every base-2 logit
// log2(e) q.k / sqrt(d) + log2 N under node u is at most U_u = (q.mu + |q| rho) log2(e) / sqrt(d)
// + lmax_u.  A block is kept if it holds a protected row (the first n1, the last n2) or if, for
// one of the G query heads of the slice, U >= m_low - tau log2(e), m_low being the best exact
// logit of the protected rows and of every block's first row.  The walk (level by level, a bit
// per visited node in LDS) evaluates a node only if its parent passed; since child balls lie in
// their parents, this keeps exactly the blocks that pass their own test.
//
// Launches of csm_index_build: index_plan, index_leaves and index_inner (described with them);
// csm_index_append: index_append.  Launches of decode_attn_logn_pruned: prune_select (one workgroup per slice: thresholds, walk,
// runs of consecutive kept blocks), prune_plan (one workgroup: the runs cut into work items and
// scanned into the item table), then the decode split and combine kernels over that table.
#include <algorithm>

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace csmkv {

constexpr int kIdxThreads = 256;
constexpr float kRadiusUp = 1.0f + 1.0f / 262144.0f;  // 1 + 2^-18

template <typename T>
__device__ __forceinline__ float elem(const char *row, int k) {
  if constexpr (__is_same(T, float)) {
    return reinterpret_cast<const float *>(row)[k];
  } else if constexpr (__is_same(T, __bf16)) {
    return bf_lo(uint32_t(reinterpret_cast<const uint16_t *>(row)[k]));
  } else {
    return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t *>(row)[k]);
  }
}

// Sum over the 64 lanes of a wave; every lane receives it.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int32_t wave_sum_i(int32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int32_t wave_max_i(int32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

struct IdxView {
  float *mu, *rho, *lmax;
  int32_t *wt;
};
__device__ __forceinline__ IdxView idx_view(const IdxArgs &a, int64_t z) {
  const int64_t nodes = 2 * (int64_t)a.P;
  return {a.mu + z * nodes * a.d, a.rho + z * nodes, a.lmax + z * nodes, a.wt + z * nodes};
}

// Centre, radius and largest log-degree of an inner node from its two children (one wave; lane l
// holds elements l + 64 e).  The caller has handled two empty children; an empty child's centre
// enters neither the centre nor the radius.
template <int EL>
__device__ __forceinline__ void combine_children(const float (&a0)[EL], const float (&a1)[EL],
                                                 int32_t w0, int32_t w1, float r0, float r1,
                                                 float l0, float l1, float (&m)[EL], float &rho,
                                                 float &lmax) {
  const float f0 = (float)w0, f1 = (float)w1, inv = 1.0f / (f0 + f1);
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    m[e] = (w0 == 0) ? a1[e] : (w1 == 0) ? a0[e] : fmaf(f0, a0[e], f1 * a1[e]) * inv;
    d0 = fmaf(a0[e] - m[e], a0[e] - m[e], d0);
    d1 = fmaf(a1[e] - m[e], a1[e] - m[e], d1);
  }
  d0 = wave_sum(d0);
  d1 = wave_sum(d1);
  float r = 0.f;
  if (w0) r = fmaxf(r, sqrtf(d0) + r0);
  if (w1) r = fmaxf(r, sqrtf(d1) + r1);
  rho = r * kRadiusUp;
  lmax = fmaxf(w0 ? l0 : -__builtin_inff(), w1 ? l1 : -__builtin_inff());
}

// Inner node u from its children in the index (one wave).  Every load of the children is issued
// before any is used, so a node costs one round trip to memory.
template <int D>
__device__ __forceinline__ void inner_node(const IdxView &v, int u, int l) {
  constexpr int EL = D / 64;
  const int c0 = 2 * u, c1 = 2 * u + 1;
  const int32_t w0 = v.wt[c0], w1 = v.wt[c1];
  const float r0 = v.rho[c0], r1 = v.rho[c1], l0 = v.lmax[c0], l1 = v.lmax[c1];
  float a0[EL], a1[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    a0[e] = v.mu[(int64_t)c0 * D + l + 64 * e];
    a1[e] = v.mu[(int64_t)c1 * D + l + 64 * e];
  }
  if (w0 + w1 == 0) {
    if (l == 0) {
      v.wt[u] = 0;
      v.rho[u] = 0.f;
      v.lmax[u] = -__builtin_inff();
    }
    return;
  }
  float m[EL], rho, lmax;
  combine_children<EL>(a0, a1, w0, w1, r0, r1, l0, l1, m, rho, lmax);
#pragma unroll
  for (int e = 0; e < EL; ++e) v.mu[(int64_t)u * D + l + 64 * e] = m[e];
  if (l == 0) {
    v.rho[u] = rho;
    v.lmax[u] = lmax;
    v.wt[u] = w0 + w1;
  }
}

// A build runs three launches.  index_plan (one workgroup) lists the non-empty leaf groups of every
// slice: kLeafGroup consecutive leaf slots (fewer when P is smaller), the leaves of one subtree.
// index_leaves (a fixed grid, two workgroups per CU, each taking groups from that list in turn):
// one wave per leaf reads the leaf's rows 16 bytes per lane (SEG lanes per row, 64 / SEG rows
// per wave load, up to 64 rows and 16 loads a pass, every load of a pass issued before any is
// used), sums the degree-weighted keys in fp32, reduces over the rows of the wave, and in a second
// pass over the same rows takes the largest distance to the centre.  A leaf that fits one pass
// keeps its rows in registers for that (its loads are then non-temporal); a longer one reads them
// again through the caches.  The workgroup then computes the inner nodes of its subtree from LDS.
// index_inner (one workgroup per slice) empties the subtrees past the slice's rows and computes
// the levels above the subtree roots.
constexpr int kLeafGroup = 8;                  // leaves per group: a subtree of height 3
constexpr int kLeafThreads = 64 * kLeafGroup;  // one wave per leaf
constexpr int kLeafGrid = 256 * 2;             // two workgroups per CU

__host__ __device__ inline int leaf_group_size(int P) { return P < kLeafGroup ? P : kLeafGroup; }

int32_t index_leaf_group(int32_t P) { return leaf_group_size(P); }

// Leaf groups of a slice of s rows (none if s is out of range: that slice's tree is empty).
__device__ __forceinline__ int slice_groups(const IdxArgs &a, int s) {
  const bool ok = s >= 0 && s <= a.max_len && (int64_t)s <= a.cap;
  const int nleaf = ok ? (s + a.B - 1) / a.B : 0;
  const int lpg = leaf_group_size(a.P);
  return (nleaf + lpg - 1) / lpg;
}

__global__ void __launch_bounds__(1024) index_plan(IdxArgs a) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x;
  const int64_t S = a.num_slices;
  const int64_t per = (S + 1023) / 1024;
  const int64_t z0 = t * per, z1 = min(S, z0 + per);
  int local = 0;
  for (int64_t z = z0; z < z1; ++z) {
    const int s = a.lens[z];
    if (!(s >= 0 && s <= a.max_len && (int64_t)s <= a.cap)) atomicExch(a.err, kDeviceError);
    local += slice_groups(a, s);
  }
  int total;
  int run = block_excl_scan<1024>(local, wsum, &total);
  for (int64_t z = z0; z < z1; ++z) {
    const int s = a.lens[z], g = slice_groups(a, s);
    for (int gi = 0; gi < g; ++gi)
      *reinterpret_cast<int4 *>(a.items + 4 * (int64_t)(run + gi)) = make_int4((int)z, gi, s, 0);
    run += g;
  }
  if (t == 0) *a.nitems = total;
}

template <typename T, int D>
__device__ __forceinline__ void seg_f32(u32x4 v, float *o) {
  if constexpr (__is_same(T, float)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  } else if constexpr (__is_same(T, __bf16)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf_lo(v[i]);
      o[2 * i + 1] = bf_hi(v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16_lo(v[i]);
      o[2 * i + 1] = f16_hi(v[i]);
    }
  }
}

// NL wave loads of a leaf's rows, STEP bytes apart, from byte soff of the leaf (AUX: the
// buffer load's cache policy bits).
template <int NL, int STEP, int AUX>
__device__ __forceinline__ void leaf_rows(u32x4 *kv, __amdgpu_buffer_rsrc_t rk, int lane_off,
                                          int soff) {
#pragma unroll
  for (int i = 0; i < NL; ++i)
    kv[i] = __builtin_bit_cast(u32x4,
                               __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + i * STEP, soff, AUX));
}

template <typename T, int D>
__global__ void __launch_bounds__(kLeafThreads) __attribute__((amdgpu_waves_per_eu(4)))
index_leaves(IdxArgs a) {
  constexpr int RB = D * (int)sizeof(T), SEG = RB / 16, RPL = 64 / SEG;  // lanes per row, rows per load
  constexpr int EPS = 16 / (int)sizeof(T);                               // elements per lane
  constexpr int NL = 64 / RPL < 16 ? 64 / RPL : 16;                     // loads per pass
  constexpr int ROWS = NL * RPL;                                         // rows per pass (<= 64)
  constexpr int EL = D / 64;
  // the subtree in heap order: node 1 its root, nodes [lpg, 2 lpg) its leaves
  __shared__ __attribute__((aligned(16))) float s_mu[2 * kLeafGroup][D];
  __shared__ float s_rho[2 * kLeafGroup], s_lmax[2 * kLeafGroup];
  __shared__ int32_t s_wt[2 * kLeafGroup];
  const int lpg = leaf_group_size(a.P);
  const int t = threadIdx.x, w = t >> 6, l = t & 63, sg = l % SEG, rw = l / SEG;
  const int total = *a.nitems;
  const int4 *items = reinterpret_cast<const int4 *>(a.items);
  int4 next = (int)blockIdx.x < total ? items[blockIdx.x] : make_int4(0, 0, 0, 0);
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    const int4 cur = next;  // (slice, group, rows)
    if (it + (int)gridDim.x < total) next = items[it + gridDim.x];
    const int64_t z = cur.x;
    const int gi = cur.y, s = cur.z;
    const int nleaf = (s + a.B - 1) / a.B;
    const IdxView v = idx_view(a, z);
    const char *Kz = a.K + z * a.cap * RB;
    const int32_t *Nz = a.N + z * a.cap;
    if (w < lpg) {
      const int b = gi * lpg + w, u = a.P + b, li = lpg + w;
      const int r0 = b * a.B, r1 = b < nleaf ? min(r0 + a.B, s) : r0;
      // the leaf's rows as range-checked buffers: rows at or past r1 read as zeros, so every
      // load is issued unconditionally
      const int nrows = __builtin_amdgcn_readfirstlane(r1 - r0);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          wave_uniform(Kz + (int64_t)r0 * RB), 0, nrows * RB, kBufWord3);
      const __amdgpu_buffer_rsrc_t rn =
          __builtin_amdgcn_make_buffer_rsrc(wave_uniform(Nz + r0), 0, nrows * 4, kBufWord3);
      const int lane_off = rw * RB + sg * 16;
      float acc[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) acc[e] = 0.f;
      int32_t W = 0, nmax = 0;
      u32x4 kv[NL];  // a leaf of at most ROWS rows stays here for pass 2
      for (int p = 0; p < nrows; p += ROWS) {  // pass 1: degree-weighted sum
        // the pass's degrees, one row per lane, handed to the lanes of each row by a shuffle
        const int32_t nrow = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rn, l < ROWS ? (p + l) * 4 : nrows * 4, 0, 0);
        if (nrows <= ROWS)  // read once: non-temporal
          leaf_rows<NL, RPL * RB, 2>(kv, rk, lane_off, p * RB);
        else  // read again in pass 2: through the caches
          leaf_rows<NL, RPL * RB, 0>(kv, rk, lane_off, p * RB);
        W += nrow;
        nmax = max(nmax, nrow);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float wi = (float)__shfl(nrow, RPL * i + rw);
          float x[EPS];
          seg_f32<T, D>(kv[i], x);
#pragma unroll
          for (int e = 0; e < EPS; ++e) acc[e] = fmaf(wi, x[e], acc[e]);
        }
      }
      // sum over the rows of the wave: lanes with the same segment hold the same elements
#pragma unroll
      for (int o = SEG; o < 64; o <<= 1) {
#pragma unroll
        for (int e = 0; e < EPS; ++e) acc[e] += __shfl_xor(acc[e], o);
      }
      W = wave_sum_i(W);
      nmax = wave_max_i(nmax);
      if (W == 0) {  // no rows, or rows of degree 0 only (they weigh nothing): an empty leaf
        if (l == 0) {
          v.wt[u] = 0;
          v.rho[u] = 0.f;
          v.lmax[u] = -__builtin_inff();
          s_wt[li] = 0;
        }
      } else {
        const float inv = 1.0f / (float)W;
        float m[EPS];
#pragma unroll
        for (int e = 0; e < EPS; ++e) m[e] = acc[e] * inv;
        if (rw == 0) {
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            v.mu[(int64_t)u * D + sg * EPS + e] = m[e];
            s_mu[li][sg * EPS + e] = m[e];
          }
        }
        float rmax = 0.f;
        const bool held = nrows <= ROWS;  // pass 1 left the leaf's rows in kv
        for (int p = 0; p < nrows; p += ROWS) {  // pass 2: the farthest row
          if (!held) leaf_rows<NL, RPL * RB, 0>(kv, rk, lane_off, p * RB);
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            float x[EPS], d2 = 0.f;
            seg_f32<T, D>(kv[i], x);
#pragma unroll
            for (int e = 0; e < EPS; ++e) d2 = fmaf(x[e] - m[e], x[e] - m[e], d2);
            d2 = lanes_sum<SEG>(d2);
            if (p + RPL * i + rw < nrows) rmax = fmaxf(rmax, d2);
          }
        }
        rmax = wave_max(rmax);
        if (l == 0) {
          const float rho = sqrtf(rmax) * kRadiusUp;
          const float lm = __builtin_amdgcn_logf((float)nmax);  // log2
          v.rho[u] = rho;
          v.lmax[u] = lm;
          v.wt[u] = W;
          s_rho[li] = rho;
          s_lmax[li] = lm;
          s_wt[li] = W;
        }
      }
    }
    __syncthreads();
    // the subtree's inner nodes: node i of a level of n nodes is global node n (P / lpg + gi) + i - n
    for (int n = lpg / 2; n >= 1; n /= 2) {
      if (w < n) {
        const int li = n + w, c0 = 2 * li, c1 = 2 * li + 1;
        const int64_t u = (int64_t)n * (a.P / lpg + gi) + w;
        const int32_t w0 = s_wt[c0], w1 = s_wt[c1];
        if (w0 + w1 == 0) {
          if (l == 0) {
            v.wt[u] = 0;
            v.rho[u] = 0.f;
            v.lmax[u] = -__builtin_inff();
            s_wt[li] = 0;
          }
        } else {
          float a0[EL], a1[EL], m[EL], rho, lmax;
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            a0[e] = s_mu[c0][l + 64 * e];
            a1[e] = s_mu[c1][l + 64 * e];
          }
          combine_children<EL>(a0, a1, w0, w1, s_rho[c0], s_rho[c1], s_lmax[c0], s_lmax[c1], m,
                               rho, lmax);
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            v.mu[u * D + l + 64 * e] = m[e];
            s_mu[li][l + 64 * e] = m[e];
          }
          if (l == 0) {
            v.rho[u] = rho;
            v.lmax[u] = lmax;
            v.wt[u] = w0 + w1;
            s_rho[li] = rho;
            s_lmax[li] = lmax;
            s_wt[li] = w0 + w1;
          }
        }
      }
      __syncthreads();
    }
  }
}

// The rest of each slice's tree, bottom-up: one workgroup per slice, a wave per node.  First the
// subtrees past the slice's last leaf group (no item of the build) are emptied; then the levels
// above the subtree roots are computed, a node whose leaves all lie at or past the slice's last
// block being empty without looking at its children.
constexpr int kInnerThreads = 1024;
template <int D>
__global__ void __launch_bounds__(kInnerThreads) index_inner(IdxArgs a) {
  const int64_t z = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const IdxView v = idx_view(a, z);
  const int s = a.lens[z];
  const bool ok = s >= 0 && s <= a.max_len && (int64_t)s <= a.cap;
  const int nleaf = ok ? (s + a.B - 1) / a.B : 0;
  const int roots = a.P / leaf_group_size(a.P), groups = slice_groups(a, s);
  for (int n = a.P; n >= roots; n /= 2) {
    for (int u = n + groups * (n / roots) + t; u < 2 * n; u += kInnerThreads) {
      v.wt[u] = 0;
      v.rho[u] = 0.f;
      v.lmax[u] = -__builtin_inff();
    }
  }
  __syncthreads();
  for (int lvl = roots / 2; lvl >= 1; lvl /= 2) {
    const int span = a.P / lvl;  // leaves under a node of this level
    for (int u = lvl + w; u < 2 * lvl; u += kInnerThreads / 64) {
      if ((u - lvl) * span >= nleaf) {
        if (l == 0) {
          v.wt[u] = 0;
          v.rho[u] = 0.f;
          v.lmax[u] = -__builtin_inff();
        }
      } else {
        inner_node<D>(v, u, l);
      }
    }
    __syncthreads();
  }
}

// One wave per slice: the row lens - 1 just appended joins its leaf; the leaf and every ancestor
// grow their radius to cover it (centres stay; an empty node takes its child's ball).
template <typename T, int D>
__global__ void __launch_bounds__(kIdxThreads) index_append(IdxArgs a) {
  constexpr int EL = D / 64, RB = D * (int)sizeof(T);
  const int64_t z = ((int64_t)blockIdx.x * kIdxThreads + threadIdx.x) >> 6;
  const int l = threadIdx.x & 63;
  if (z >= a.num_slices) return;
  const int s = a.lens[z];
  if (s < 1 || (int64_t)s > a.cap) {
    if (s != 0 && l == 0) atomicExch(a.err, kDeviceError);
    return;
  }
  const IdxView v = idx_view(a, z);
  const int r = s - 1, b = r / a.B;
  const char *row = a.K + (z * a.cap + r) * RB;
  const int32_t n = a.N[z * a.cap + r];
  int u = a.P + b;
  float k[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) k[e] = elem<T>(row, l + 64 * e);
  const float ln = __builtin_amdgcn_logf((float)n);
  // every lane computes the same radius and log-degree; lane 0 stores them, and the walk up uses
  // the register copies (each lane reads back only centre elements it owns)
  float rc, lc;
  if (r % a.B == 0) {  // a new leaf: its centre is the row
#pragma unroll
    for (int e = 0; e < EL; ++e) v.mu[(int64_t)u * D + l + 64 * e] = k[e];
    rc = 0.f;
    lc = ln;
    if (l == 0) v.wt[u] = n;
  } else {
    float d2 = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const float x = k[e] - v.mu[(int64_t)u * D + l + 64 * e];
      d2 = fmaf(x, x, d2);
    }
    d2 = wave_sum(d2);
    rc = fmaxf(v.rho[u], sqrtf(d2) * kRadiusUp);
    lc = fmaxf(v.lmax[u], ln);
    if (l == 0) v.wt[u] = v.wt[u] + n;
  }
  if (l == 0) {
    v.rho[u] = rc;
    v.lmax[u] = lc;
  }
  while (u > 1) {
    const int p = u / 2;
    const int32_t wp = v.wt[p];
    float rp, lp;
    if (wp == 0) {  // an empty ancestor takes its child's ball
#pragma unroll
      for (int e = 0; e < EL; ++e)
        v.mu[(int64_t)p * D + l + 64 * e] = v.mu[(int64_t)u * D + l + 64 * e];
      rp = rc;
      lp = lc;
    } else {
      float d2 = 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const float x = v.mu[(int64_t)u * D + l + 64 * e] - v.mu[(int64_t)p * D + l + 64 * e];
        d2 = fmaf(x, x, d2);
      }
      d2 = wave_sum(d2);
      rp = fmaxf(v.rho[p], (sqrtf(d2) + rc) * kRadiusUp);
      lp = fmaxf(v.lmax[p], lc);
    }
    if (l == 0) {
      v.rho[p] = rp;
      v.lmax[p] = lp;
      v.wt[p] = wp + n;
    }
    rc = rp;
    lc = lp;
    u = p;
  }
}

// acc[h] += <x, q_h> over D elements: x a row of the storage type (16-byte loads, all issued
// before use) or an fp32 centre (float4 loads); q_h in LDS.
template <typename T, int G, int D>
__device__ __forceinline__ void dot_row(const char *row, const float (*s_q)[D], float *acc) {
  // BAT 16-byte loads in flight at a time, in at least two batches (with one, every q index
  // is a constant and the compiler holds all of q in registers)
  constexpr int EPS = 16 / (int)sizeof(T), NS = D / EPS, BAT = NS / 2 < 8 ? NS / 2 : 8;
#pragma unroll 1
  for (int i0 = 0; i0 < NS; i0 += BAT) {
    u32x4 seg[BAT];
#pragma unroll
    for (int i = 0; i < BAT; ++i) seg[i] = ld16(row + 16 * (i0 + i));
#pragma unroll
    for (int i = 0; i < BAT; ++i) {
      float x[EPS];
      seg_f32<T, D>(seg[i], x);
#pragma unroll
      for (int e = 0; e < EPS; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(x[e], s_q[h][EPS * (i0 + i) + e], acc[h]);
    }
  }
}

// One workgroup per slice: thresholds from the reference rows, the walk, the runs of kept blocks.
// Trees of at most kEagerNodes nodes have every node's test evaluated in one parallel pass and
// are then walked over the resulting bits (a leaf is kept when it and every ancestor passed: the
// same set as the level-by-level walk, whose dependent loads per level it avoids); larger trees
// are walked level by level, evaluating only the nodes whose parent passed.
constexpr int kSelThreads = 512;
constexpr int kEagerNodes = 4096;
template <typename T, int G, int D>
__global__ void __launch_bounds__(kSelThreads) prune_select(IdxArgs a) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int NW = kSelThreads / 64;
  __shared__ float s_q[G][D], s_qn[G], s_th[NW][G];
  __shared__ uint32_t s_vis[2][kPruneMaxLeaves / 32];
  __shared__ uint32_t s_pass[kEagerNodes / 32];
  __shared__ int32_t s_cnt[NW], s_cnt2[NW];
  const int64_t z = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int64_t g = z / a.H_kv, kvh = z % a.H_kv;
  const int s = a.lens[z];
  const bool ok = s >= 0 && s <= a.max_len && (int64_t)s <= a.cap;
  const IdxView v = idx_view(a, z);
  int32_t *runs = a.runs + z * (int64_t)a.max_runs * 2;
  if (!ok || s == 0) {
    if (!ok && t == 0) atomicExch(a.err, kDeviceError);
    if (t == 0) a.nruns[z] = 0;
    return;
  }
  const int nleaf = (s + a.B - 1) / a.B;
  for (int i = t; i < G * D; i += kSelThreads) {
    const int h = i / D, k = i % D;
    s_q[h][k] = elem<T>(a.q + ((g * a.H_q + kvh * G + h) * (int64_t)D) * sizeof(T), k);
  }
  __syncthreads();
  if (w == 0) {
    for (int h = 0; h < G; ++h) {
      float x = 0.f;
      for (int k = l; k < D; k += 64) x = fmaf(s_q[h][k], s_q[h][k], x);
      x = wave_sum(x);
      if (l == 0) s_qn[h] = sqrtf(x);
    }
  }
  // m_low: exact logits of the protected rows and of every block's first row
  const char *Kz = a.K + z * a.cap * RB;
  const int32_t *Nz = a.N + z * a.cap;
  const int p0 = min(a.n1, s), p1 = max(s - a.n2, 0);
  const int nref = p0 + (s - p1) + nleaf;
  float best[G];
#pragma unroll
  for (int h = 0; h < G; ++h) best[h] = -__builtin_inff();
#pragma unroll 1
  for (int i = t; i < nref; i += kSelThreads) {
    const int r = i < p0 ? i : i < p0 + (s - p1) ? p1 + (i - p0) : (i - p0 - (s - p1)) * a.B;
    const char *row = Kz + (int64_t)r * RB;
    const float ln = __builtin_amdgcn_logf((float)Nz[r]);
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    dot_row<T, G, D>(row, s_q, acc);
#pragma unroll
    for (int h = 0; h < G; ++h) best[h] = fmaxf(best[h], fmaf(acc[h], a.scale_log2, ln));
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = wave_max(best[h]);
    if (l == 0) s_th[w][h] = m;
  }
  const int pw = (a.P + 31) / 32;  // words of a level's bits
  const bool eager = 2 * a.P <= kEagerNodes;
  for (int i = t; i < pw; i += kSelThreads) s_vis[0][i] = s_vis[1][i] = 0u;
  if (eager)
    for (int i = t; i < (2 * a.P + 31) / 32; i += kSelThreads) s_pass[i] = 0u;
  __syncthreads();
  float th[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = s_th[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) m = fmaxf(m, s_th[ww][h]);
    th[h] = m - a.tau_log2;
  }
  // a node's test: its bound reaches the threshold for one of the heads (empty nodes never pass)
  auto passes = [&](int u) {
    const float rr = v.rho[u], lm = v.lmax[u];
    float dq[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dq[h] = 0.f;
    dot_row<float, G, D>(reinterpret_cast<const char *>(v.mu + (int64_t)u * D), s_q, dq);
    bool pass = false;
#pragma unroll
    for (int h = 0; h < G; ++h) pass |= fmaf(fmaf(s_qn[h], rr, dq[h]), a.scale_log2, lm) >= th[h];
    return pass;
  };
  int cur = 0;
  if (eager) {
#pragma unroll 1
    for (int u = 1 + t; u < 2 * a.P; u += kSelThreads)
      if (v.wt[u] > 0 && passes(u)) atomicOr(&s_pass[u >> 5], 1u << (u & 31));
    __syncthreads();
    for (int b = t; b < a.P; b += kSelThreads) {  // the walk over the bits, from the leaf up
      bool k = true;
      for (int u = a.P + b; u >= 1 && k; u >>= 1) k = (s_pass[u >> 5] >> (u & 31)) & 1u;
      if (k) atomicOr(&s_vis[1][b >> 5], 1u << (b & 31));
    }
    __syncthreads();
  } else {
    // the walk: level `span` holds nodes [span, 2 span); a visited node that passes marks its
    // children (next level) visited, or, at the leaves, keeps its block
    if (t == 0 && v.wt[1] > 0) s_vis[0][0] = 1u;  // the root, bit 0 of level 1
    __syncthreads();
    for (int span = 1; span <= a.P; span *= 2) {
      const bool leaves = span == a.P;
#pragma unroll 1
      for (int i = t; i < span; i += kSelThreads) {
        if (!((s_vis[cur][i >> 5] >> (i & 31)) & 1u)) continue;
        const int u = span + i;
        if (!passes(u)) continue;
        if (leaves) {
          atomicOr(&s_vis[cur ^ 1][i >> 5], 1u << (i & 31));  // reused below as the kept set
        } else {
          for (int c = 0; c < 2; ++c)
            if (v.wt[2 * u + c] > 0)
              atomicOr(&s_vis[cur ^ 1][(2 * i + c) >> 5], 1u << ((2 * i + c) & 31));
        }
      }
      __syncthreads();
      if (!leaves) {
        for (int i = t; i < pw; i += kSelThreads) s_vis[cur][i] = 0u;
        cur ^= 1;
        __syncthreads();
      }
    }
  }
  uint32_t *kept = s_vis[cur ^ 1];
  // blocks with a protected row are kept
  for (int b = t; b < nleaf; b += kSelThreads) {
    const int r0 = b * a.B, r1 = min(r0 + a.B, s);
    if (r0 < p0 || r1 > p1) atomicOr(&kept[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  if (a.kept_tap != nullptr)
    for (int b = t; b < a.P; b += kSelThreads)
      a.kept_tap[z * a.P + b] = b < nleaf ? (uint8_t)((kept[b >> 5] >> (b & 31)) & 1u) : 0;
  // runs of consecutive kept blocks, in order: a run starts at a kept block whose predecessor is
  // not kept and ends at a kept block whose successor is not; the k-th start and the k-th end
  // belong to one run.  Each thread takes a contiguous range of blocks; two scans over the
  // threads give every start and every end its rank.
  const int per = (nleaf + kSelThreads - 1) / kSelThreads, b0 = t * per, b1 = min(nleaf, b0 + per);
  auto kb = [&](int b) { return b >= 0 && b < nleaf && ((kept[b >> 5] >> (b & 31)) & 1u); };
  int ns = 0, ne = 0;
  for (int b = b0; b < b1; ++b) {
    const bool k = kb(b);
    ns += k && !kb(b - 1);
    ne += k && !kb(b + 1);
  }
  int is = ns, ie = ne;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ys = __shfl_up(is, o), ye = __shfl_up(ie, o);
    if (l >= o) {
      is += ys;
      ie += ye;
    }
  }
  if (l == 63) {
    s_cnt[w] = is;
    s_cnt2[w] = ie;
  }
  __syncthreads();
  int bs = 0, be = 0;
  for (int ww = 0; ww < w; ++ww) {
    bs += s_cnt[ww];
    be += s_cnt2[ww];
  }
  int ks = bs + is - ns, ke = be + ie - ne;
  for (int b = b0; b < b1; ++b) {
    const bool k = kb(b);
    if (k && !kb(b - 1)) runs[2 * ks++] = b * a.B;
    if (k && !kb(b + 1)) runs[2 * ke++ + 1] = min((b + 1) * a.B, s);
  }
  if (t == kSelThreads - 1) a.nruns[z] = bs + is;
}

// One workgroup: every slice's runs cut into work items of at most tsplit tokens (a run of r
// tokens into ceil(r / tsplit) items whose lengths differ by at most one), scanned into the item
// table and the per-slice item offsets the decode split and combine kernels read.
__global__ void __launch_bounds__(1024) prune_plan(IdxArgs a) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t S = a.num_slices;
  const int64_t per = (S + 1023) / 1024;
  const int64_t z0 = t * per, z1 = min(S, z0 + per);
  const int ts = a.tsplit;
  int local = 0;
  for (int64_t z = z0; z < z1; ++z) {
    const int32_t *runs = a.runs + z * (int64_t)a.max_runs * 2;
    for (int k = 0; k < a.nruns[z]; ++k) local += (runs[2 * k + 1] - runs[2 * k] + ts - 1) / ts;
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int run = 0, total = 0;
  for (int i = 0; i < 16; ++i) {
    run += i < w ? wsum[i] : 0;
    total += wsum[i];
  }
  run += incl - local;
  for (int64_t z = z0; z < z1; ++z) {
    a.item_off[z] = run;
    const int32_t *runs = a.runs + z * (int64_t)a.max_runs * 2;
    for (int k = 0; k < a.nruns[z]; ++k) {
      const int r0 = runs[2 * k], len = runs[2 * k + 1] - r0, cnt = (len + ts - 1) / ts;
      const int q = len / cnt, rem = len - q * cnt;
      for (int p = 0; p < cnt; ++p)
        *reinterpret_cast<int4 *>(a.item_zp + 4 * (int64_t)(run + p)) =
            make_int4((int)z, r0 + p * q + min(p, rem), r0 + (p + 1) * q + min(p + 1, rem), 0);
      run += cnt;
    }
  }
  if (t == 1023) a.item_off[S] = total;
}

template <typename T, int D>
static int launch_idx_t(const IdxArgs &a, int op, hipStream_t st) {
  if (op == 0) {
    hipLaunchKernelGGL(index_plan, dim3(1), dim3(1024), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const int64_t items = a.num_slices * (a.P / leaf_group_size(a.P));
    const uint32_t grid = (uint32_t)std::min<int64_t>(items, kLeafGrid);
    hipLaunchKernelGGL((index_leaves<T, D>), dim3(grid), dim3(kLeafThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL((index_inner<D>), dim3((uint32_t)a.num_slices), dim3(kInnerThreads), 0, st, a);
  } else
    hipLaunchKernelGGL((index_append<T, D>), dim3((uint32_t)((a.num_slices * 64 + kIdxThreads - 1) / kIdxThreads)),
                       dim3(kIdxThreads), 0, st, a);
  return (int)hipGetLastError();
}

int launch_index(const IdxArgs &a, int dtype, int d, int op, hipStream_t st) {
  if (a.num_slices == 0) return 0;
  if (d == 64)
    return dtype == kDtypeF32 ? launch_idx_t<float, 64>(a, op, st)
           : dtype == kDtypeF16 ? launch_idx_t<_Float16, 64>(a, op, st)
                                : launch_idx_t<__bf16, 64>(a, op, st);
  return dtype == kDtypeF32 ? launch_idx_t<float, 128>(a, op, st)
         : dtype == kDtypeF16 ? launch_idx_t<_Float16, 128>(a, op, st)
                              : launch_idx_t<__bf16, 128>(a, op, st);
}

template <typename T, int D>
static int launch_select_t(const IdxArgs &a, int G, hipStream_t st) {
  const dim3 grid((uint32_t)a.num_slices), blk(kSelThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((prune_select<T, 1, D>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prune_select<T, 2, D>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((prune_select<T, 4, D>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((prune_select<T, 8, D>), grid, blk, 0, st, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_prune(const IdxArgs &a, int dtype, int d, int G, hipStream_t st) {
  if (a.num_slices == 0) return 0;
  int rc;
  if (d == 64)
    rc = dtype == kDtypeF32 ? launch_select_t<float, 64>(a, G, st)
         : dtype == kDtypeF16 ? launch_select_t<_Float16, 64>(a, G, st)
                              : launch_select_t<__bf16, 64>(a, G, st);
  else
    rc = dtype == kDtypeF32 ? launch_select_t<float, 128>(a, G, st)
         : dtype == kDtypeF16 ? launch_select_t<_Float16, 128>(a, G, st)
                              : launch_select_t<__bf16, 128>(a, G, st);
  if (rc) return rc;
  hipLaunchKernelGGL(prune_plan, dim3(1), dim3(1024), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace csmkv
