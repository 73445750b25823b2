// One round of Chunked Soft Matching (CSM) over every slice of a K/V cache.
//
// Method: Chelsea review, section 三, 分块软匹配算法 steps 1-4 (chunking with protected sink
// and recent tokens, alternating A/B partition, soft matching, merge into one centre
// per cluster with degree n_t) and Algorithm 1 (K, V, N, s rewritten by a round);
// CentroidKV page, 分块软匹配 (CSM) (cosine similarity, each A token takes its most
// similar B token, top fraction r of the ranked matches merged) and 聚合 (degree-weighted
// averaging of K and V; degrees accumulate over rounds).
//
// Launch structure (all on the caller's stream):
//   csm_prep   : validates every lens[] entry (a bad one sets the sticky error word), decides which
//                slices run (all, or those at their trigger threshold) and with which r,
//                records each slice's input and output length, resets the per-slice
//                ticket counters and clears the per-chunk "source consumed" flags.
//   csm_round  : one workgroup per unit (512 threads for chunks of up to 256 rows, 256 for
//                fp32 storage at d = 128, 1024 for chunks of up to 512 rows); units are (slice,
//                chunk) pairs plus one "tail" unit per slice that moves the recent rows and
//                writes lens.  A workgroup's slice comes from its block index (a slice that does
//                not run exits at once, touching no counter); its unit within the slice is a
//                ticket from that slice's atomic counter, so every lower-numbered unit of the
//                slice has already started when a unit runs.
//
// In-place compaction: chunk j of a slice writes rows [n1 + j*(c - m), ...), which may
// overlap the source rows of chunks i <= j.  A chunk loads its whole source (K, V, N)
// into LDS and registers, waits for its loads to land, and raises its flag; before
// writing it waits for the flags of the lower chunks whose sources its destination
// overlaps.  Those chunks hold lower tickets of the same slice, are already running and
// raise their flag without waiting on anything, so every wait ends (a bounded poll turns a
// wait that does not end into the sticky error word).  Lower chunks never write into a higher
// chunk's source.
//
// Per chunk (A = even offsets, B = odd; up to 128 of each for c <= 256, 256 for c <= 512; head
// dim d = 64 or 128):
//   keys -> LDS tile (swizzled rows), reciprocal fp32 norms from the same registers; values
//   stay in registers;
//   S^T = B_keys . A_keys^T on MFMA (16-bit: v_mfma_f32_32x32x16_bf16 / _f16, fp32:
//   v_mfma_f32_32x32x2_f32): the waves split the tile into 32-column A groups times B parts;
//   cosine = (dot * fl(1/max(|b|,1e-12))) * fl(1/max(|a|,1e-12)) in fp32, branch-free arg-max
//   per A column inside each lane, then across the two half-waves, then across the B parts
//   through LDS (lowest B index on ties);
//   rank of every A edge by (score desc, index asc) from unique 64-bit keys, a comparison count
//   split over all threads;
//   per-target source lists in ascending A order: same-target lanes found with ballots over the
//   target index bits, slots by mbcnt, counts scanned across targets;
//   keep-mask prefix sum (ballot + mbcnt) gives each kept row its output slot;
//   rows that are not merge targets are copied in one pass; merge targets, compacted into
//   a list, are computed as (N_b k_b + sum N_a k_a) * rcp(N_b + sum N_a) in fp32 and
//   stored rounded to nearest even; values pass through the same LDS tile after the keys;
//   stores are non-temporal (the output is not re-read by the round).
#include <algorithm>

#include "csm_common.hpp"
#include "device_common.hpp"
#include "kernel_args.hpp"

namespace csmkv {


__global__ void csm_prep(CsmArgs a) {
  if (blockIdx.x == 0) {
    for (int64_t z = threadIdx.x; z < a.num_slices; z += blockDim.x) {
      const int s = a.lens_in[z];
      const bool outl = a.mask != nullptr && a.mask[z] != 0;
      bool ok = s >= 0 && (int64_t)s <= a.cap_in;
      // Algorithm 1 trigger (when thresholds are given): cluster when s >= B + g.  An outlier
      // slice in place is neither read nor written, so it needs no cover by the launch.
      const bool run = !(outl && a.in_place) && (a.thr == nullptr || (ok && !outl && s >= a.thr[z]));
      if (run && s > a.max_len) ok = false;  // the launch covers max_len rows
      double r = a.r;
      if (a.thr != nullptr && run && ok) {  // r annealed over this slice's rounds
        const int j = a.round_idx[z];
        r = fmax(__dsub_rn(a.r_init, __dmul_rn((double)j, a.r_delta)), a.r_min);
        a.round_idx[z] = j + 1;
      }
      int s_new = s;
      const int M = s - a.n1 - a.n2;
      if (ok && run && !outl && M >= 2) {
        const int nch = (M + a.c - 1) / a.c;
        const int last = M - (nch - 1) * a.c;
        s_new = s - (nch - 1) * merge_count_dev(r, a.c) - merge_count_dev(r, last);
      }
      if (ok && (int64_t)s_new > a.cap_out) ok = false;
      a.s_in[z] = ok ? s : -1;
      a.s_out[z] = s_new;
      a.s_r[z] = run && ok ? r : -1.0;  // the round's workgroups exit on this one load
      a.ticket[z] = 0u;
      if (!ok) atomicExch(a.err, kDeviceError);
    }
  } else {
    const int64_t total = a.num_slices * (int64_t)a.units;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)(gridDim.x - 1) * blockDim.x)
      a.flags[i] = 0;
  }
}

template <typename T, int NT, int D>
__device__ void tail_unit(const CsmArgs &a, int64_t z, int s, int s_new, int nch, bool outl) {
  using TL = Tile<T, NT, D>;
  const int t = threadIdx.x;
  const int64_t kin = z * a.cap_in * TL::ROWB, kout = z * a.cap_out * TL::ROWB;
  const char *Ks = a.Kin + kin, *Vs = a.Vin + kin;
  const int32_t *Ns = a.Nin + z * a.cap_in;
  char *Kd = a.Kout + kout, *Vd = a.Vout + kout;
  int32_t *Nd = a.Nout + z * a.cap_out;
  int32_t *src = a.tap_src ? a.tap_src + z * a.cap_out : nullptr;
  if (nch == 0) {  // nothing to compress: lens unchanged, copy everything out of place
    if (!a.in_place) copy_rows<T, NT, D>(Ks, Vs, Ns, Kd, Vd, Nd, s);
    if (src)
      for (int i = t; i < s; i += blockDim.x) src[i] = i;
    if (t == 0) a.lens_out[z] = s;
    return;
  }
  const int n1 = a.n1, n2 = a.n2, c = a.c;
  __shared__ int s_stuck;
  if (!a.in_place) copy_rows<T, NT, D>(Ks, Vs, Ns, Kd, Vd, Nd, n1);
  if (t == 0) s_stuck = 0;
  if (a.in_place && !outl && t == 0) {
    // the recent rows land in [s_new - n2, s_new): wait for chunks whose sources overlap it
    const int d0 = s_new - n2, d1 = s_new;
    if (d1 > d0) {
      const int lo = (d0 - n1) / c, hi = min(nch - 1, (d1 - 1 - n1) / c);
      bool ok = true;
      for (int i = lo; i <= hi && ok; ++i) ok = wait_flag(a.flags + z * a.units + i);
      if (!ok) {  // a wait that did not end: report it and leave the rows unwritten
        atomicExch(a.err, kDeviceError);
        s_stuck = 1;
      }
    }
  }
  __syncthreads();
  if (s_stuck) return;
  const int64_t so = (int64_t)(s - n2), dof = (int64_t)(s_new - n2);
  copy_rows<T, NT, D>(Ks + so * TL::ROWB, Vs + so * TL::ROWB, Ns + so, Kd + dof * TL::ROWB,
               Vd + dof * TL::ROWB, Nd + dof, n2);
  if (src) {
    for (int i = t; i < n1; i += blockDim.x) src[i] = i;
    for (int i = t; i < n2; i += blockDim.x) src[s_new - n2 + i] = s - n2 + i;
  }
  if (t == 0) a.lens_out[z] = s_new;
}

// Unique 64-bit key ordering A edges by descending score, then ascending index: the score's
// bits mapped to an order-preserving unsigned integer (-0 folded into +0), then 255 - a.
__device__ __forceinline__ uint64_t rank_key(float score, int aidx) {
  const uint32_t u = __float_as_uint(score + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 8) | (uint64_t)(255 - aidx);
}

// One unit of the round.  T: storage type; NT: threads; D: head dim; CMAX: chunk capacity
// (256: A and B up to 128 rows; 512: up to 256).  NA = CMAX / 2 A rows; the A x B tile is
// split over the waves as AG = NA / 32 column groups times NT / 64 / AG B parts.
template <typename T, int NT, int D, int CMAX>
__device__ __forceinline__ void csm_round_body(const CsmArgs &a) {
  using TL = Tile<T, NT, D, CMAX>;
  constexpr int ROWB = TL::ROWB, SEGS = TL::SEGS, RPI = TL::RPI, NLD = TL::NLD, EPS = TL::EPS;
  constexpr int NA = CMAX / 2;       // A (and B) rows per chunk at most
  constexpr int NW = NT / 64;        // waves
  constexpr int AG = NA / 32;        // 32-column A groups
  constexpr int BP = NW / AG;        // B parts (waves per A group)
  constexpr int BT = AG / BP;        // 32-row B tiles per wave
  // B tiles per MFMA pass (bounds the live accumulators; d = 64 kernels run at 6 waves/SIMD)
  constexpr int TP = (BT < 2 || D == 64) ? 1 : 2;
  constexpr int NQ = NT / NA;        // parts of the rank count
  constexpr int LW = NA / 64;        // waves holding the A rows in the list step
  constexpr int TBITS = NA == 128 ? 7 : 8;  // bits of a target index
  constexpr int OW = CMAX / 64;      // waves covering the output slots
  static_assert(NT >= CMAX && BP >= 1 && AG % BP == 0 && BT % TP == 0, "tile split");
  static_assert(NA == 128 || NA == 256, "chunk capacity 256 or 512");
  __shared__ __attribute__((aligned(16))) char tile[CMAX * ROWB];
  __shared__ __attribute__((aligned(16))) float s_invA[NA], s_invB[NA];  // 1 / max(|k|, eps)
  __shared__ int32_t s_n[CMAX];
  __shared__ int32_t s_outrow[CMAX];
  __shared__ int32_t s_best[NA], s_sel[NA], s_cnt[NA], s_wsum[NA], s_off[NA], s_list[NA];
  __shared__ int32_t s_cntw[LW][NA], s_rank[NQ][NA];
  __shared__ int32_t s_mrg[OW][64], s_mcnt[OW];
  __shared__ __attribute__((aligned(16))) uint64_t s_key[NA];  // rank keys, 0 = no edge
  __shared__ float s_bsc[BP][NA];  // per B part: best score and index of every A row
  __shared__ int32_t s_bix[BP][NA];
  __shared__ int32_t s_misc[1 + NW];

  const int t = threadIdx.x;
  const int64_t z = blockIdx.x / (uint32_t)a.units;
  // r < 0: the slice does not run this call (trigger not met, outlier in place, or a bad length
  // with the error word already set) and is left as it is; one load decides it
  const double r = a.s_r[z];
  if (r < 0.0) return;
  const int s = a.s_in[z];
  if (s < 0) return;
  const bool outl = a.mask != nullptr && a.mask[z] != 0;
  if (outl && a.in_place) return;
  if (t == 0) s_misc[0] = (int32_t)atomicAdd(a.ticket + z, 1u);
  __syncthreads();
  const int u = s_misc[0];
  const int n1 = a.n1, n2 = a.n2, c = a.c;
  const int m_full = merge_count_dev(r, c);
  const int M = s - n1 - n2;
  const int nch = M >= 2 ? (M + c - 1) / c : 0;
  const int s_new = a.s_out[z];

  if (u == a.units - 1) {
    tail_unit<T, NT, D>(a, z, s, s_new, nch, outl);
    return;
  }
  if (u >= nch) return;

  // ---------------------------------------------------------------- chunk unit
  const int j = u;
  const int start = n1 + j * c;
  const int L = min(c, M - j * c);
  const bool copy_only = outl;  // outlier slice, out of place: rows move unchanged
  const int m = copy_only ? 0 : merge_count_dev(r, L);
  const int nA = (L + 1) / 2, nB = L / 2;
  const int base = copy_only ? start : n1 + j * (c - m_full);
  const int nout = L - m;
  T *tsel = nullptr;

  const char *Ksrc = a.Kin + (z * a.cap_in + start) * (int64_t)ROWB;
  const char *Vsrc = a.Vin + (z * a.cap_in + start) * (int64_t)ROWB;
  const int sg = t % SEGS, r0 = t / SEGS;

  // 1. load the chunk: keys first, then degrees, then values.  The load counter retires in
  //    order, so the key tile (+ norms) is written as soon as the keys land while the
  //    values are still in flight; they are only needed for the output.
  u32x4 vreg[NLD];
  {
    u32x4 kreg[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = r0 + RPI * i;
      kreg[i] = r < L ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4 *>(Ksrc + (int64_t)r * ROWB + sg * 16))
                      : u32x4{0u, 0u, 0u, 0u};
    }
    const int32_t nval = t < L ? a.Nin[z * a.cap_in + start + t] : 0;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = r0 + RPI * i;
      vreg[i] = r < L ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4 *>(Vsrc + (int64_t)r * ROWB + sg * 16))
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = r0 + RPI * i;
      *reinterpret_cast<u32x4 *>(tile + lds_swz(r, sg, ROWB)) = kreg[i];
      const float ss = lanes_sum<SEGS>(seg_sumsq(kreg[i], tsel));
      if (sg == 0) {
        const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
        if (r & 1) s_invB[r >> 1] = inv; else s_invA[r >> 1] = inv;
      }
    }
    if (t < L) s_n[t] = nval;
  }
  __syncthreads();

  // 2. similarity tile on MFMA and arg-max over B for every A column.  Wave w holds A
  //    columns [32 (w mod AG), +32) against the BT B tiles of part w / AG, TP tiles per MFMA
  //    pass; with several B parts the parts are merged through LDS (a lower part holds lower
  //    B indices and wins ties).
  if (!copy_only && nB > 0) {
    const int w = t >> 6, l = t & 63, h = l >> 5, col = l & 31;
    const int bq = w / AG;
    const int aidx = 32 * (w % AG) + col;
    const float ia = s_invA[aidx];
    float best = -__builtin_inff();
    int bidx = 0;
#pragma unroll
    for (int tp = 0; tp < BT; tp += TP) {
      f32x16 acc[TP];
#pragma unroll
      for (int tl = 0; tl < TP; ++tl)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[tl][q] = 0.f;
      sim_tile<TP, D>(tile, aidx, col, h, acc, tsel, bq * BT + tp);
      // cosine = (dot * (1/|b|)) * (1/|a|); lowest B index wins a tie (ascending, strict >)
#pragma unroll
      for (int tl = 0; tl < TP; ++tl) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int b0 = (bq * BT + tp + tl) * 32 + 8 * g4 + 4 * h;
          const float4 ib = *reinterpret_cast<const float4 *>(&s_invB[b0]);
          const float ibv[4] = {ib.x, ib.y, ib.z, ib.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sc = (acc[tl][4 * g4 + i] * ibv[i]) * ia;
            sc = (b0 + i < nB) ? sc : -__builtin_inff();
            const bool up = sc > best;
            best = up ? sc : best;
            bidx = up ? b0 + i : bidx;
          }
        }
      }
    }
    const float ob = __shfl_xor(best, 32);
    const int oi = __shfl_xor(bidx, 32);
    if (ob > best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
    if (h == 0) {
      if (BP == 1) {
        s_best[aidx] = aidx < nA ? bidx : -1;
        s_key[aidx] = aidx < nA ? rank_key(best, aidx) : 0ull;
      } else {
        s_bsc[bq][aidx] = best;
        s_bix[bq][aidx] = bidx;
      }
    }
  } else if (t < NA) {
    s_best[t] = -1;
    s_key[t] = 0ull;
  }
  // in place: every load of this chunk has landed before its "source consumed" flag rises
  if (a.in_place) wait_vm_loads();
  __syncthreads();
  if (a.in_place && t == 0)
    __hip_atomic_store(a.flags + z * a.units + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (BP > 1) {
    if (!copy_only && nB > 0 && t < NA) {
      float best = s_bsc[0][t];
      int bidx = s_bix[0][t];
#pragma unroll
      for (int p = 1; p < BP; ++p) {
        const float sc = s_bsc[p][t];
        const bool up = sc > best;
        best = up ? sc : best;
        bidx = up ? s_bix[p][t] : bidx;
      }
      s_best[t] = t < nA ? bidx : -1;
      s_key[t] = t < nA ? rank_key(best, t) : 0ull;
    }
    __syncthreads();
  }

  // 3. top-m selection: rank of each A edge by (score desc, index asc), i.e. the number of
  //    larger unique keys.  Every thread counts over one of NQ parts of the NA candidates.
  {
    constexpr int PART = NA / NQ;
    const int aa = t % NA, part = t / NA;
    const uint64_t my = s_key[aa];
    int cnt = 0;
#pragma unroll 8
    for (int q = part * PART; q < part * PART + PART; q += 2) {
      const uint64_t k0 = s_key[q], k1 = s_key[q + 1];
      cnt += (k0 > my) + (k1 > my);
    }
    s_rank[part][aa] = cnt;
  }
  __syncthreads();
  if (t < NA) {
    int rank = 0;
#pragma unroll
    for (int p = 0; p < NQ; ++p) rank += s_rank[p][t];
    s_sel[t] = (t < nA && m > 0 && nB > 0) ? (rank < m) : 0;
#pragma unroll
    for (int w = 0; w < LW; ++w) s_cntw[w][t] = 0;
    s_wsum[t] = t < nB ? s_n[2 * t + 1] : 0;
  }
  __syncthreads();

  // 4. source lists.  Waves 0 .. LW-1 hold the A rows, 64 each; lanes with the same target
  //    are found with TBITS ballots over the bits of the target index, which gives each
  //    source its slot among the same-target sources of its wave (ascending A).
  int my_pos = 0, my_b = -1;
  if (t < NA) {
    const int aa = t;
    const bool sa = s_sel[aa] != 0;
    const int b = sa ? s_best[aa] : 0;
    uint64_t eq = __ballot(sa);
#pragma unroll
    for (int bit = 0; bit < TBITS; ++bit) {
      const uint64_t mb = __ballot(sa && ((b >> bit) & 1));
      eq &= ((b >> bit) & 1) ? mb : ~mb;
    }
    if (sa) {
      my_b = b;
      my_pos = lanes_below(eq);
      if (my_pos == 0) s_cntw[t >> 6][b] = __popcll(eq);
      atomicAdd(&s_wsum[b], s_n[2 * aa]);
    }
  }
  const int keep = (t < L) && ((t & 1) || !s_sel[t >> 1]);
  const uint64_t bal = __ballot(keep);
  const int pre = lanes_below(bal);
  if ((t & 63) == 0) s_misc[1 + (t >> 6)] = __popcll(bal);
  __syncthreads();
  if (t < 64) {  // per-target counts and their exclusive scan (NA / 64 targets per lane)
    constexpr int TPL = NA / 64;
    int cnt[TPL], tot = 0;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      int cc = 0;
#pragma unroll
      for (int w = 0; w < LW; ++w) cc += s_cntw[w][TPL * t + k];
      cnt[k] = cc;
      tot += cc;
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (t >= o) incl += y;
    }
    int ex = incl - tot;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      s_off[TPL * t + k] = ex;
      s_cnt[TPL * t + k] = cnt[k];
      ex += cnt[k];
    }
  }
  {
    int off = 0;
    for (int w = 0; w < (t >> 6); ++w) off += s_misc[1 + w];
    if (keep) s_outrow[off + pre] = t;
  }
  __syncthreads();
  if (my_b >= 0) {
    int before = 0;  // same-target sources of the lower waves come first
    for (int w = 0; w < (t >> 6); ++w) before += s_cntw[w][my_b];
    s_list[s_off[my_b] + before + my_pos] = t;
  }
  if (t < CMAX) {  // output slots that hold a merged target, compacted per wave
    bool mg = false;
    if (t < nout) {
      const int r = s_outrow[t];
      mg = (r & 1) && s_cnt[r >> 1] > 0;
    }
    const uint64_t mb = __ballot(mg);
    if (mg) s_mrg[t >> 6][lanes_below(mb)] = t;
    if ((t & 63) == 0) s_mcnt[t >> 6] = __popcll(mb);
  }
  if (a.in_place && t == 0) {
    // destination rows [base, base + nout) overlap the sources of chunks lo..j
    const int lo = (base - n1) / c, hi = min(j - 1, (base + nout - 1 - n1) / c);
    bool ok = true;
    for (int i = lo; i <= hi && ok; ++i) ok = wait_flag(a.flags + z * a.units + i);
    if (!ok) {  // a wait that did not end: report it and leave the chunk's rows unwritten
      atomicExch(a.err, kDeviceError);
      s_misc[0] = -1;
    }
  }
  __syncthreads();
  if (s_misc[0] == -1) return;

  if (a.tap_best != nullptr && t < NA) {
    const int64_t o = (z * a.units + j) * NA + t;
    a.tap_best[o] = (t < nA && !copy_only) ? s_best[t] : -1;
    a.tap_sel[o] = (uint8_t)s_sel[t];
  }
  if (a.tap_src != nullptr && t < nout) a.tap_src[z * a.cap_out + base + t] = start + s_outrow[t];

  // 5. write K (merged rows averaged in fp32), then V through the same LDS tile, then N
  char *Kdst = a.Kout + (z * a.cap_out + base) * (int64_t)ROWB;
  char *Vdst = a.Vout + (z * a.cap_out + base) * (int64_t)ROWB;
  int nmerged = 0;
#pragma unroll
  for (int w = 0; w < OW; ++w) nmerged += s_mcnt[w];
  for (int pass = 0; pass < 2; ++pass) {
    char *dst = pass == 0 ? Kdst : Vdst;
    if (pass == 1) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        *reinterpret_cast<u32x4 *>(tile + lds_swz(r0 + RPI * i, sg, ROWB)) = vreg[i];
      __syncthreads();
    }
    // rows that are not merge targets move unchanged
#pragma unroll 4
    for (int i = 0; i < NLD; ++i) {
      const int p = r0 + RPI * i;
      if (p >= nout) break;
      const int r = s_outrow[p];
      if ((r & 1) && s_cnt[r >> 1] > 0) continue;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(tile + lds_swz(r, sg, ROWB)),
                                  reinterpret_cast<u32x4 *>(dst + (int64_t)p * ROWB + sg * 16));
    }
    // merge targets: (N_b x_b + sum N_a x_a) * (1 / W), fp32, sources in ascending A order
    for (int idx = r0; idx < nmerged; idx += RPI) {
      int wv = 0, rem = idx;  // the wave list holding merged slot idx, and its position
#pragma unroll
      for (int w = 0; w < OW - 1; ++w) {
        const int cw = s_mcnt[w];
        const bool past = wv == w && rem >= cw;
        rem -= past ? cw : 0;
        wv += past ? 1 : 0;
      }
      const int p = s_mrg[wv][rem];
      const int r = s_outrow[p];
      const int b = r >> 1;
      float accv[EPS], tmp[EPS];
      seg_unpack(*reinterpret_cast<const u32x4 *>(tile + lds_swz(r, sg, ROWB)), tmp, tsel);
      const float nb = (float)s_n[r];
#pragma unroll
      for (int e = 0; e < EPS; ++e) accv[e] = nb * tmp[e];
      const int q0 = s_off[b], q1 = q0 + s_cnt[b];
      for (int q = q0; q < q1; ++q) {
        const int ar = 2 * s_list[q];
        const float wa = (float)s_n[ar];
        seg_unpack(*reinterpret_cast<const u32x4 *>(tile + lds_swz(ar, sg, ROWB)), tmp, tsel);
#pragma unroll
        for (int e = 0; e < EPS; ++e) accv[e] = fmaf(wa, tmp[e], accv[e]);
      }
      const float inv = __builtin_amdgcn_rcpf((float)s_wsum[b]);  // v_rcp_f32, 1 ulp
#pragma unroll
      for (int e = 0; e < EPS; ++e) accv[e] *= inv;
      __builtin_nontemporal_store(seg_pack(accv, tsel),
                                  reinterpret_cast<u32x4 *>(dst + (int64_t)p * ROWB + sg * 16));
    }
  }
  if (t < nout) {
    const int r = s_outrow[t];
    const int b = r >> 1;
    a.Nout[z * a.cap_out + base + t] = ((r & 1) && s_cnt[b] > 0) ? s_wsum[b] : s_n[r];
  }
}

// Head dim 128.  bf16 / fp16: 512 threads and 78 KB of LDS per workgroup, two workgroups
// (four waves per SIMD) per CU.  fp32: the 128 KB key tile allows one workgroup per CU.
constexpr int kWideThreads = 512;
constexpr int kBigThreads = 1024;
__global__ void __launch_bounds__(kWideThreads, 2) csm_round_bf16(CsmArgs a) {
  csm_round_body<__bf16, kWideThreads, 128, kMaxChunk>(a);
}
__global__ void __launch_bounds__(kWideThreads, 2) csm_round_f16(CsmArgs a) {
  csm_round_body<_Float16, kWideThreads, 128, kMaxChunk>(a);
}
__global__ void __launch_bounds__(256, 1) csm_round_f32(CsmArgs a) {
  csm_round_body<float, 256, 128, kMaxChunk>(a);
}
// Head dim 64: half the tile.  bf16 / fp16: 46 KB of LDS, so three 512-thread workgroups fit
// a CU when a thread holds at most 85 VGPRs (six waves per SIMD); fp32: 79 KB, two per CU.
__global__ void __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(6, 8)))
csm_round_bf16_d64(CsmArgs a) {
  csm_round_body<__bf16, kWideThreads, 64, kMaxChunk>(a);
}
__global__ void __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(6, 8)))
csm_round_f16_d64(CsmArgs a) {
  csm_round_body<_Float16, kWideThreads, 64, kMaxChunk>(a);
}
__global__ void __launch_bounds__(kWideThreads, 2) csm_round_f32_d64(CsmArgs a) {
  csm_round_body<float, kWideThreads, 64, kMaxChunk>(a);
}
// Chunks up to 512 rows (256 x 256 similarity tile), bf16 / fp16: 1024 threads, one workgroup
// per CU (the d = 128 key tile is 128 KB).
__global__ void __launch_bounds__(kBigThreads, 1) csm_round_bf16_c512(CsmArgs a) {
  csm_round_body<__bf16, kBigThreads, 128, kMaxChunkWide>(a);
}
__global__ void __launch_bounds__(kBigThreads, 1) csm_round_f16_c512(CsmArgs a) {
  csm_round_body<_Float16, kBigThreads, 128, kMaxChunkWide>(a);
}
__global__ void __launch_bounds__(kBigThreads, 1) csm_round_bf16_d64_c512(CsmArgs a) {
  csm_round_body<__bf16, kBigThreads, 64, kMaxChunkWide>(a);
}
__global__ void __launch_bounds__(kBigThreads, 1) csm_round_f16_d64_c512(CsmArgs a) {
  csm_round_body<_Float16, kBigThreads, 64, kMaxChunkWide>(a);
}

// Host-side launcher used by the C ABI (d is 64 or 128; c <= 512, and c <= 256 for fp32).
// Returns 0 or a hipError_t value.
int launch_csm(const CsmArgs &args, int dtype, int d, hipStream_t stream) {
  const int64_t total = args.num_slices * (int64_t)args.units;
  const int prep_blocks = 1 + (int)std::min<int64_t>(1024, (total + 255) / 256);
  hipLaunchKernelGGL(csm_prep, dim3(prep_blocks), dim3(256), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (total == 0) return 0;
  const dim3 grid((uint32_t)total), wide(kWideThreads), big(kBigThreads);
  const bool f32 = dtype == kDtypeF32, f16 = dtype == kDtypeF16;
  if (args.c > kMaxChunk) {
    if (f32) return (int)hipErrorInvalidValue;  // rejected by the C ABI before this point
    if (d == 64) {
      if (f16) hipLaunchKernelGGL(csm_round_f16_d64_c512, grid, big, 0, stream, args);
      else hipLaunchKernelGGL(csm_round_bf16_d64_c512, grid, big, 0, stream, args);
    } else {
      if (f16) hipLaunchKernelGGL(csm_round_f16_c512, grid, big, 0, stream, args);
      else hipLaunchKernelGGL(csm_round_bf16_c512, grid, big, 0, stream, args);
    }
  } else if (d == 64) {
    if (f32) hipLaunchKernelGGL(csm_round_f32_d64, grid, wide, 0, stream, args);
    else if (f16) hipLaunchKernelGGL(csm_round_f16_d64, grid, wide, 0, stream, args);
    else hipLaunchKernelGGL(csm_round_bf16_d64, grid, wide, 0, stream, args);
  } else {
    if (f32) hipLaunchKernelGGL(csm_round_f32, grid, dim3(256), 0, stream, args);
    else if (f16) hipLaunchKernelGGL(csm_round_f16, grid, wide, 0, stream, args);
    else hipLaunchKernelGGL(csm_round_bf16, grid, wide, 0, stream, args);
  }
  e = hipGetLastError();
  return (int)e;
}

}  // namespace csmkv
