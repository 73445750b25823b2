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
//                fp32 storage at d = 128, 1024 for chunks of up to 512 rows; at r <= 1/2 with
//                16-bit storage the register-resident kernels, 256 threads for chunks of up to
//                256 rows at d = 128 and for chunks of up to 512 rows); units are (slice,
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
//   keys -> LDS tile (swizzled rows; the register-resident kernels stage only the B keys and
//   load the A keys into MFMA operand registers), reciprocal fp32 norms from the same
//   registers; values stay in registers;
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

// ROWS: rows per block of the copies (see copy_rows).
template <typename T, int NT, int D, int ROWS = kMaxChunk>
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
    if (!a.in_place) copy_rows<T, NT, D, ROWS>(Ks, Vs, Ns, Kd, Vd, Nd, s);
    if (src)
      for (int i = t; i < s; i += blockDim.x) src[i] = i;
    if (t == 0) a.lens_out[z] = s;
    return;
  }
  const int n1 = a.n1, n2 = a.n2, c = a.c;
  __shared__ int s_stuck;
  if (!a.in_place) copy_rows<T, NT, D, ROWS>(Ks, Vs, Ns, Kd, Vd, Nd, n1);
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
  copy_rows<T, NT, D, ROWS>(Ks + so * TL::ROWB, Vs + so * TL::ROWB, Ns + so, Kd + dof * TL::ROWB,
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

// One chunk unit of a slice, as the workgroup's ticket assigns it.
struct ChunkUnit {
  int64_t z;       // slice
  int j;           // chunk of the slice
  int start, L;    // first source row, rows in the chunk
  int m, nA, nB;   // merges, A rows, B rows
  int base, nout;  // first output row, output rows
  bool copy_only;  // outlier slice out of place: its rows move unchanged
};

// Starts a workgroup of the round: a slice that does not run this call (r < 0: trigger not met,
// outlier in place, or a bad length with the error word already set) is left as it is, one load
// deciding it; otherwise the workgroup takes a ticket from its slice's counter (slot: one int of
// LDS), runs the slice's tail unit if the ticket names it, and returns true with cu filled in when
// the ticket names a chunk.  ROWS: rows per block of the tail unit's copies.
template <typename T, int NT, int D, int ROWS>
__device__ __forceinline__ bool take_unit(const CsmArgs &a, int32_t *slot, ChunkUnit &cu) {
  const int64_t z = blockIdx.x / (uint32_t)a.units;
  const double r = a.s_r[z];
  if (r < 0.0) return false;
  const int s = a.s_in[z];
  if (s < 0) return false;
  const bool outl = a.mask != nullptr && a.mask[z] != 0;
  if (outl && a.in_place) return false;
  if (threadIdx.x == 0) *slot = (int32_t)atomicAdd(a.ticket + z, 1u);
  __syncthreads();
  const int u = *slot;
  const int n1 = a.n1, n2 = a.n2, c = a.c;
  const int M = s - n1 - n2;
  const int nch = M >= 2 ? (M + c - 1) / c : 0;
  if (u == a.units - 1) {
    tail_unit<T, NT, D, ROWS>(a, z, s, a.s_out[z], nch, outl);
    return false;
  }
  if (u >= nch) return false;
  cu.z = z;
  cu.j = u;
  cu.start = n1 + u * c;
  cu.L = min(c, M - u * c);
  cu.copy_only = outl;
  cu.m = outl ? 0 : merge_count_dev(r, cu.L);
  cu.nA = (cu.L + 1) / 2;
  cu.nB = cu.L / 2;
  cu.base = outl ? cu.start : n1 + u * (c - merge_count_dev(r, c));
  cu.nout = cu.L - cu.m;
  return true;
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
  ChunkUnit cu;
  if (!take_unit<T, NT, D, kMaxChunk>(a, &s_misc[0], cu)) return;
  const int64_t z = cu.z;
  const int j = cu.j, start = cu.start, L = cu.L, m = cu.m, nA = cu.nA, nB = cu.nB;
  const int base = cu.base, nout = cu.nout, n1 = a.n1, c = a.c;
  const bool copy_only = cu.copy_only;
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

// MFMA step for 16-bit keys: acc += B rows (32 x 16, from LDS) . A rows^T (16 x 32, registers).
__device__ __forceinline__ f32x16 mfma16(u32x4 b, u32x4 a, f32x16 acc, __bf16 *) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                 __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma16(u32x4 b, u32x4 a, f32x16 acc, _Float16 *) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b),
                                                __builtin_bit_cast(f16x8, a), acc, 0, 0, 0);
}

// One unit of the round for chunks of up to CMAX rows when at most a quarter of the rows merge
// (r <= 1/2), on NT threads: one per A row (256 for chunks of up to 512 rows: two workgroups per
// CU at d = 128, three at d = 64) or two (256 for chunks of up to 256 rows: three workgroups per
// CU at d = 128).  The steps and every decision and rounding are those of csm_round_body; what
// differs is where the rows live.  The A keys go from memory straight into MFMA operand
// registers (wave w holds A groups GPW w .. GPW w + GPW - 1, lane (col, h) segments 2k + h of its
// A row, as the LDS tile feeds them in csm_round_body), only the B keys are staged in LDS, and
// the values stay in registers.  At output, unmerged A keys and values are stored from
// registers; the rows that take part in a merge go through the B-key tile: a target keeps its B
// slot, and since at most a quarter of a chunk's rows are sources there are at least as many B
// rows that are not targets as there are sources, so the j-th source (ascending A) takes the
// j-th such slot once that row has been written out.
template <typename T, int D, int CMAX, int NT>
__device__ __forceinline__ void csm_round_regs_body(const CsmArgs &a) {
  constexpr int NA = CMAX / 2, NW = NT / 64;
  constexpr int GPW = NA / 32 / NW;  // A groups of 32 rows per wave
  constexpr int LW = NA / 64;        // waves that hold the A rows in the list step
  static_assert(NT == NA || NT == 2 * NA, "one or two threads per A row");
  constexpr int ROWB = D * (int)sizeof(T), SEGS = ROWB / 16, KS = D / 16, SWM = SEGS - 1;
  constexpr int RPI = NT / SEGS;    // rows per block-wide load (16 lanes a row at d = 128)
  constexpr int NLB = NA / RPI;     // loads per thread for the B rows
  constexpr int NLV = CMAX / RPI;   // loads per thread for every row
  constexpr int EPS = 16 / (int)sizeof(T);
  // Value loads issued before the similarity (the rest right after it): all of them at d = 64 or
  // with one A group per wave; with two groups per wave at d = 128 only half fit beside the A
  // keys and the MFMA accumulators.
  constexpr int VE = (D == 64 || GPW == 1) ? NLV : NLV / 2;
  // Where the "source consumed" flag rises, once every load of the chunk has landed: after the
  // similarity (0), or after the rank (1) when values were still loading during the similarity.
  // Either way it rises before the chunk waits for any other chunk's flag.
  constexpr int FLAG_AT = VE == NLV ? 0 : 1;
  static_assert(sizeof(T) == 2 && (D == 64 || D == 128), "16-bit storage, d = 64 or 128");
  static_assert(CMAX == kMaxChunk || CMAX == kMaxChunkWide, "chunk capacity 256 or 512");
  static_assert(NA % 64 == 0 && NA <= 256, "whole waves of A rows; 8-bit target indices");
  struct SimPart {
    uint64_t key[NA];  // rank keys, 0 = no edge
    float invB[NA];    // 1 / max(|k_b|, eps)
  };
  struct OutPart {
    int32_t list[NA];  // sources of every target, by target, ascending A
    int32_t tgt[NA];   // merge targets (B indices)
    int32_t src[NA];   // tile row holding each source A row
    int32_t fre[NA];   // B rows that are not targets, ascending
  };
  struct __attribute__((aligned(16))) Smem {
    char tile[NA * ROWB];
    union {
      SimPart s;
      OutPart o;
    } u1;
    union {
      int32_t cntw[LW][NA];  // same-target counts of each wave that holds A rows
      int32_t slot[CMAX];    // output row of every kept row
    } u2;
    int32_t n[CMAX];
    int32_t best[NA], sel[NA], cnt[NA], wsum[NA], off[NA];
    int32_t misc[1 + 5 * NW];
  };
  __shared__ Smem sm;
  auto swzb = [](int b, int seg) { return b * ROWB + ((seg ^ (b & SWM)) << 4); };
  // LDS offset of this thread's segment of B row rb + RPI i: the swizzle repeats every PER values
  // of i, so PER base addresses serve them all
  static_assert(RPI % SEGS == 0 || SEGS % RPI == 0, "swizzle period");
  constexpr int PER = RPI >= SEGS ? 1 : SEGS / RPI;
  const int rb0 = threadIdx.x / SEGS, sg0 = threadIdx.x % SEGS;
  auto bslot = [=](int i) {
    return swzb(rb0 + RPI * (i % PER), sg0) + (i - i % PER) * RPI * ROWB;
  };

  const int t = threadIdx.x;
  ChunkUnit cu;
  // 128-row blocks in the tail unit's copies: fewer live registers
  if (!take_unit<T, NT, D, 128>(a, &sm.misc[0], cu)) return;
  const int64_t z = cu.z;
  const int j = cu.j, start = cu.start, L = cu.L, m = cu.m, nA = cu.nA, nB = cu.nB;
  const int base = cu.base, nout = cu.nout, n1 = a.n1, c = a.c;
  const bool copy_only = cu.copy_only;
  T *tsel = nullptr;
  const char *Ksrc = a.Kin + (z * a.cap_in + start) * (int64_t)ROWB;
  const char *Vsrc = a.Vin + (z * a.cap_in + start) * (int64_t)ROWB;
  const int w = t >> 6, l = t & 63, col = l & 31, h = l >> 5;
  const int sg = t % SEGS, rb = t / SEGS;

  // 1. loads: A keys into operand registers, B keys into the tile (+ their norms), degrees,
  //    then the values.  A keys use cached loads: each 128-byte line is read by four of a
  //    lane's loads, issued back to back.
  // range-checked buffers over the chunk's L rows: rows past them read as zeros
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(wave_uniform(Ksrc), 0, L * ROWB, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(wave_uniform(Vsrc), 0, L * ROWB, kBufWord3);
  u32x4 areg[GPW][KS];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int voff = 2 * (32 * (GPW * w + gi) + col) * ROWB + h * 16;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      areg[gi][kk] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff + kk * 32, 0, 0));
  }
  {
    u32x4 breg[NLB];
    const int voff = (2 * rb + 1) * ROWB + sg * 16;
#pragma unroll
    for (int i = 0; i < NLB; ++i)
      breg[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, 2 * RPI * ROWB * i, 2));
    const int32_t *Nsrc = a.Nin + z * a.cap_in + start;
    const int32_t nv0 = t < L ? Nsrc[t] : 0, nv1 = t + NT < L ? Nsrc[t + NT] : 0;
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
      *reinterpret_cast<u32x4 *>(sm.tile + bslot(i)) = breg[i];
      const float ss = lanes_sum<SEGS>(seg_sumsq(breg[i], tsel));
      if (sg == 0) sm.u1.s.invB[rb + RPI * i] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
    }
    sm.n[t] = nv0;
    if (t + NT < CMAX) sm.n[t + NT] = nv1;
  }
  // A norms, summed in the order of the 16-lane tree of the B norms: segment pairs (2k, 2k+1)
  // first (one from each half-wave), then pairs of pairs
  float ia[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    float p[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const float x = seg_sumsq(areg[gi][kk], tsel);
      p[kk] = x + __shfl_xor(x, 32);
    }
    float ss;
    if constexpr (KS == 8)
      ss = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    else
      ss = (p[0] + p[1]) + (p[2] + p[3]);
    ia[gi] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  }
  u32x4 vreg[NLV];
  const int voffv = rb * ROWB + sg * 16;
#pragma unroll
  for (int i = 0; i < VE; ++i)
    vreg[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voffv, RPI * ROWB * i, 2));
  __syncthreads();

  // 2. similarity and arg-max over B (ascending B, strict >, lowest index on ties); both A
  //    groups of the wave against one B tile at a time (one operand read, two MFMA chains)
  if (!copy_only && nB > 0) {
    float best[GPW];
    int bidx[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      best[gi] = -__builtin_inff();
      bidx[gi] = 0;
    }
#pragma unroll 1
    for (int bt = 0; bt < NA / 32; ++bt) {
      f32x16 acc[GPW];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[gi][q] = 0.f;
      const char *brow = sm.tile + bt * 32 * ROWB;  // rows bt 32 + col share col's swizzle
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4 braw = *reinterpret_cast<const u32x4 *>(brow + swzb(col, 2 * kk + h));
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) acc[gi] = mfma16(braw, areg[gi][kk], acc[gi], tsel);
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int b0 = bt * 32 + 8 * g4 + 4 * h;
        const float4 ib = *reinterpret_cast<const float4 *>(&sm.u1.s.invB[b0]);
        const float ibv[4] = {ib.x, ib.y, ib.z, ib.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi) {
            float sc = (acc[gi][4 * g4 + i] * ibv[i]) * ia[gi];
            sc = (b0 + i < nB) ? sc : -__builtin_inff();
            const bool up = sc > best[gi];
            best[gi] = up ? sc : best[gi];
            bidx[gi] = up ? b0 + i : bidx[gi];
          }
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int aidx = 32 * (GPW * w + gi) + col;
      const float ob = __shfl_xor(best[gi], 32);
      const int oi = __shfl_xor(bidx[gi], 32);
      if (ob > best[gi] || (ob == best[gi] && oi < bidx[gi])) {
        best[gi] = ob;
        bidx[gi] = oi;
      }
      if (h == 0) {
        sm.best[aidx] = aidx < nA ? bidx[gi] : -1;
        sm.u1.s.key[aidx] = aidx < nA ? rank_key(best[gi], aidx) : 0ull;
      }
    }
  } else if (t < NA) {
    sm.best[t] = -1;
    sm.u1.s.key[t] = 0ull;
  }
  // the remaining values, in flight through the rank and list steps
#pragma unroll
  for (int i = VE; i < NLV; ++i)
    vreg[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voffv, RPI * ROWB * i, 2));
  // in place: every load of this chunk has landed before its "source consumed" flag rises
  if (FLAG_AT == 0 && a.in_place) wait_vm_loads();
  __syncthreads();
  if (FLAG_AT == 0 && a.in_place && t == 0)
    __hip_atomic_store(a.flags + z * a.units + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 3. top-m selection: rank of each A edge = number of larger unique keys
  if (t < NA) {
    const uint64_t my = sm.u1.s.key[t];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < NA; q += 2) {
      const uint64_t k0 = sm.u1.s.key[q], k1 = sm.u1.s.key[q + 1];
      rank += (k0 > my) + (k1 > my);
    }
    sm.sel[t] = (t < nA && m > 0 && nB > 0) ? (rank < m) : 0;
#pragma unroll
    for (int ww = 0; ww < LW; ++ww) sm.u2.cntw[ww][t] = 0;
    sm.wsum[t] = t < nB ? sm.n[2 * t + 1] : 0;
  }
  if (FLAG_AT == 1 && a.in_place) wait_vm_loads();
  __syncthreads();
  if (FLAG_AT == 1 && a.in_place && t == 0)
    __hip_atomic_store(a.flags + z * a.units + j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 4. source lists (ballots over the 8 target-index bits), kept rows, targets, free B rows
  const bool sa = t < NA && sm.sel[t] != 0;
  int my_pos = 0, my_b = -1;
  {
    const int b = sa ? sm.best[t] : 0;
    uint64_t eq = __ballot(sa);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t mb = __ballot(sa && ((b >> bit) & 1));
      eq &= ((b >> bit) & 1) ? mb : ~mb;
    }
    if (sa) {
      my_b = b;
      my_pos = lanes_below(eq);
      if (my_pos == 0) sm.u2.cntw[w][b] = __popcll(eq);
      atomicAdd(&sm.wsum[b], sm.n[2 * t]);
    }
  }
  const bool keep0 = t < L && ((t & 1) || !sm.sel[t >> 1]);
  const bool keep1 = t + NT < L && (((t + NT) & 1) || !sm.sel[(t + NT) >> 1]);
  const uint64_t bal0 = __ballot(keep0), bal1 = __ballot(keep1);
  if (l == 0) {
    sm.misc[1 + w] = __popcll(bal0);
    sm.misc[1 + NW + w] = __popcll(bal1);
  }
  __syncthreads();
  if (t < 64) {  // per-target counts and their exclusive scan (NA / 64 targets per lane)
    constexpr int TPL = NA / 64;
    int cn[TPL], tot = 0;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      int cc = 0;
#pragma unroll
      for (int ww = 0; ww < LW; ++ww) cc += sm.u2.cntw[ww][TPL * t + k];
      cn[k] = cc;
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
      sm.off[TPL * t + k] = ex;
      sm.cnt[TPL * t + k] = cn[k];
      ex += cn[k];
    }
  }
  __syncthreads();
  if (my_b >= 0) {
    int before = 0;  // same-target sources of the lower waves come first
    for (int ww = 0; ww < w; ++ww) before += sm.u2.cntw[ww][my_b];
    sm.u1.o.list[sm.off[my_b] + before + my_pos] = t;
  }
  const bool is_tgt = t < nB && sm.cnt[t] > 0;
  const bool is_free = t < nB && sm.cnt[t] == 0;
  const uint64_t btg = __ballot(is_tgt), bfr = __ballot(is_free), bsr = __ballot(sa);
  if (l == 0) {
    sm.misc[1 + 2 * NW + w] = __popcll(btg);
    sm.misc[1 + 3 * NW + w] = __popcll(bfr);
    sm.misc[1 + 4 * NW + w] = __popcll(bsr);
  }
  if (a.in_place && t == 0) {
    // destination rows [base, base + nout) overlap the sources of chunks lo..j
    const int lo = (base - n1) / c, hi = min(j - 1, (base + nout - 1 - n1) / c);
    bool ok = true;
    for (int i = lo; i <= hi && ok; ++i) ok = wait_flag(a.flags + z * a.units + i);
    if (!ok) {  // a wait that did not end: report it and leave the chunk's rows unwritten
      atomicExch(a.err, kDeviceError);
      sm.misc[0] = -1;
    }
  }
  __syncthreads();
  if (sm.misc[0] == -1) return;
  int slot0 = 0, slot1 = 0, srank = 0, ntgt = 0;
  {
    int o0 = 0, o1 = 0, ot = 0, of = 0, tot0 = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const bool lower = ww < w;
      tot0 += sm.misc[1 + ww];
      ntgt += sm.misc[1 + 2 * NW + ww];
      o0 += lower ? sm.misc[1 + ww] : 0;
      o1 += lower ? sm.misc[1 + NW + ww] : 0;
      ot += lower ? sm.misc[1 + 2 * NW + ww] : 0;
      of += lower ? sm.misc[1 + 3 * NW + ww] : 0;
      srank += lower ? sm.misc[1 + 4 * NW + ww] : 0;
    }
    slot0 = o0 + lanes_below(bal0);
    slot1 = tot0 + o1 + lanes_below(bal1);
    srank += lanes_below(bsr);
    if (keep0) sm.u2.slot[t] = slot0;
    if (keep1) sm.u2.slot[t + NT] = slot1;
    if (is_tgt) sm.u1.o.tgt[ot + lanes_below(btg)] = t;
    if (is_free) sm.u1.o.fre[of + lanes_below(bfr)] = t;
  }
  __syncthreads();
  if (sa) sm.u1.o.src[t] = sm.u1.o.fre[srank];
  if (a.tap_best != nullptr && t < NA) {
    const int64_t o = (z * a.units + j) * NA + t;
    a.tap_best[o] = (t < nA && !copy_only) ? sm.best[t] : -1;
    a.tap_sel[o] = (uint8_t)sm.sel[t];
  }
  if (a.tap_src != nullptr) {
    int32_t *ts = a.tap_src + z * a.cap_out + base;
    if (keep0) ts[slot0] = start + t;
    if (keep1) ts[slot1] = start + t + NT;
  }
  __syncthreads();

  // 5. keys: B rows that are not targets from the tile, unmerged A rows from the registers;
  //    then the sources into the freed B rows and the merged rows
  //    (N_b k_b + sum N_a k_a) * (1 / W) in fp32, sources in ascending A order
  // output rows [0, nout) of the chunk's destination, as range-checked buffers
  const __amdgpu_buffer_rsrc_t rko = __builtin_amdgcn_make_buffer_rsrc(
      wave_uniform(a.Kout + (z * a.cap_out + base) * (int64_t)ROWB), 0, nout * ROWB, kBufWord3);
  const __amdgpu_buffer_rsrc_t rvo = __builtin_amdgcn_make_buffer_rsrc(
      wave_uniform(a.Vout + (z * a.cap_out + base) * (int64_t)ROWB), 0, nout * ROWB, kBufWord3);
  auto store_row_seg = [](const __amdgpu_buffer_rsrc_t &rs, u32x4 v, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 2);  // non-temporal
  };
  auto merge_rows = [&](const __amdgpu_buffer_rsrc_t &dst) {
    for (int idx = rb; idx < ntgt; idx += RPI) {
      const int b = sm.u1.o.tgt[idx];
      float accv[EPS], tmp[EPS];
      seg_unpack(*reinterpret_cast<const u32x4 *>(sm.tile + swzb(b, sg)), tmp, tsel);
      const float nb = (float)sm.n[2 * b + 1];
#pragma unroll
      for (int e = 0; e < EPS; ++e) accv[e] = nb * tmp[e];
      const int q0 = sm.off[b], q1 = q0 + sm.cnt[b];
      for (int q = q0; q < q1; ++q) {
        const int aa = sm.u1.o.list[q];
        const float wa = (float)sm.n[2 * aa];
        seg_unpack(*reinterpret_cast<const u32x4 *>(sm.tile + swzb(sm.u1.o.src[aa], sg)), tmp,
                   tsel);
#pragma unroll
        for (int e = 0; e < EPS; ++e) accv[e] = fmaf(wa, tmp[e], accv[e]);
      }
      const float inv = __builtin_amdgcn_rcpf((float)sm.wsum[b]);  // v_rcp_f32, 1 ulp
#pragma unroll
      for (int e = 0; e < EPS; ++e) accv[e] *= inv;
      store_row_seg(dst, seg_pack(accv, tsel), sm.u2.slot[2 * b + 1] * ROWB + sg * 16);
    }
  };
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int b = rb + RPI * i;
    if (b < nB && sm.cnt[b] == 0)
      store_row_seg(rko, *reinterpret_cast<const u32x4 *>(sm.tile + bslot(i)),
                    sm.u2.slot[2 * b + 1] * ROWB + sg * 16);
  }
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int aidx = 32 * (GPW * w + gi) + col;
    if (aidx < nA && !sm.sel[aidx]) {
      const int off = sm.u2.slot[2 * aidx] * ROWB + h * 16;
      // cached stores: a lane writes 16 of every 32 bytes of its row, and its partner lane the
      // rest; the lines stay in L2 until both halves are in, so each reaches memory once
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        __builtin_amdgcn_raw_buffer_store_b128(areg[gi][kk], rko, off + kk * 32, 0, 0);
    }
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int aidx = 32 * (GPW * w + gi) + col;
    if (aidx < nA && sm.sel[aidx]) {
      const int fs = sm.u1.o.src[aidx];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        *reinterpret_cast<u32x4 *>(sm.tile + swzb(fs, 2 * kk + h)) = areg[gi][kk];
    }
  }
  __syncthreads();
  merge_rows(rko);
  __syncthreads();

  // 6. values: rows that take part in a merge into the tile as the keys were, the others
  //    straight from the registers; then the merged rows; then N
#pragma unroll
  for (int i = 0; i < NLV; ++i) {
    const int rr = rb + RPI * i;
    if (rr < L) {
      const int hb = rr >> 1;
      int trow = -1;
      if (rr & 1) trow = sm.cnt[hb] > 0 ? hb : -1;
      else trow = sm.sel[hb] ? sm.u1.o.src[hb] : -1;
      if (trow >= 0)
        *reinterpret_cast<u32x4 *>(sm.tile + swzb(trow, sg)) = vreg[i];
      else
        store_row_seg(rvo, vreg[i], sm.u2.slot[rr] * ROWB + sg * 16);
    }
  }
  __syncthreads();
  merge_rows(rvo);
  int32_t *Nd = a.Nout + z * a.cap_out + base;
  if (keep0) Nd[slot0] = ((t & 1) && sm.cnt[t >> 1] > 0) ? sm.wsum[t >> 1] : sm.n[t];
  if (keep1) Nd[slot1] = (((t + NT) & 1) && sm.cnt[(t + NT) >> 1] > 0) ? sm.wsum[(t + NT) >> 1]
                                                                        : sm.n[t + NT];
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
// Chunks up to 512 rows at r <= 1/2, 16-bit storage: A keys and values in registers, one thread
// per A row (256).  d = 128: 79 KB of LDS and up to 256 registers a lane, two workgroups per CU;
// d = 64: 47 KB, three per CU.  (For chunks up to 256 rows the same body on 128 threads, four
// workgroups per CU at d = 128, is no faster than csm_round_body's two 512-thread workgroups.)
constexpr int kRegsThreads = 256;
#define CSMKV_REGS_KERNEL(NAME, T, D, CMAX, NT, WPE)                                         \
  __global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))           \
  NAME(CsmArgs a) {                                                                          \
    csm_round_regs_body<T, D, CMAX, NT>(a);                                                  \
  }
CSMKV_REGS_KERNEL(csm_round_bf16_c512_regs, __bf16, 128, kMaxChunkWide, 256, 2)
CSMKV_REGS_KERNEL(csm_round_f16_c512_regs, _Float16, 128, kMaxChunkWide, 256, 2)
CSMKV_REGS_KERNEL(csm_round_bf16_d64_c512_regs, __bf16, 64, kMaxChunkWide, 256, 3)
CSMKV_REGS_KERNEL(csm_round_f16_d64_c512_regs, _Float16, 64, kMaxChunkWide, 256, 3)
CSMKV_REGS_KERNEL(csm_round_bf16_regs, __bf16, 128, kMaxChunk, 256, 3)
CSMKV_REGS_KERNEL(csm_round_f16_regs, _Float16, 128, kMaxChunk, 256, 3)
#undef CSMKV_REGS_KERNEL

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
    if (args.r <= 0.5) {  // args.r bounds every slice's r, annealed r included
      const dim3 regs(kRegsThreads);
      if (d == 64) {
        if (f16) hipLaunchKernelGGL(csm_round_f16_d64_c512_regs, grid, regs, 0, stream, args);
        else hipLaunchKernelGGL(csm_round_bf16_d64_c512_regs, grid, regs, 0, stream, args);
      } else {
        if (f16) hipLaunchKernelGGL(csm_round_f16_c512_regs, grid, regs, 0, stream, args);
        else hipLaunchKernelGGL(csm_round_bf16_c512_regs, grid, regs, 0, stream, args);
      }
    } else if (d == 64) {
      if (f16) hipLaunchKernelGGL(csm_round_f16_d64_c512, grid, big, 0, stream, args);
      else hipLaunchKernelGGL(csm_round_bf16_d64_c512, grid, big, 0, stream, args);
    } else {
      if (f16) hipLaunchKernelGGL(csm_round_f16_c512, grid, big, 0, stream, args);
      else hipLaunchKernelGGL(csm_round_bf16_c512, grid, big, 0, stream, args);
    }
  } else if (!f32 && d == 128 && args.r <= 0.5) {
    const dim3 regs(kRegsThreads);
    if (f16) hipLaunchKernelGGL(csm_round_f16_regs, grid, regs, 0, stream, args);
    else hipLaunchKernelGGL(csm_round_bf16_regs, grid, regs, 0, stream, args);
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
