// Argument blocks and host launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csmkv {

struct CsmArgs {
  const char *Kin, *Vin;
  const int32_t *Nin;
  char *Kout, *Vout;
  int32_t *Nout;
  int32_t *lens_out;
  const int32_t *lens_in;
  const uint8_t *mask;
  int64_t num_slices, cap_in, cap_out;
  int32_t max_len, n1, n2, c, units, in_place;
  double r;
  // device-side trigger (nullable thr: every slice runs with r)
  const int32_t *thr;   // [num_slices] a slice runs when its length >= thr[z]
  int32_t *round_idx;   // [num_slices] rounds run so far; r = max(r_init - j * r_delta, r_min)
  double r_init, r_delta, r_min;
  // workspace
  int32_t *err;      // sticky device error word (set on a bad length, never cleared here)
  uint32_t *ticket;  // [num_slices] unit ticket counters
  int32_t *s_in;     // [num_slices] validated input length, -1 = skip the slice
  int32_t *s_out;    // [num_slices] output length
  double *s_r;       // [num_slices] this round's r, < 0 = slice not clustered this call
  int32_t *flags;    // [num_slices][units] "chunk source consumed"
  // debug taps (nullable)
  int32_t *tap_best;
  uint8_t *tap_sel;
  int32_t *tap_src;
};

struct DecArgs {
  const char *q, *K, *V;
  const int32_t *N, *lens;
  float *O;
  int64_t num_slices, cap;
  int32_t max_len, H_q, H_kv;
  int32_t tsplit;     // tokens per work item of the plan kernel (dec_split_tokens)
  float scale_log2;   // log2(e) / sqrt(d)
  int32_t *err;       // sticky device error word (set on a bad length, never cleared here)
  int32_t *item_off;  // [num_slices + 1] first work item of each slice (plan kernel only)
  int32_t *s_in;      // [num_slices] each length as the plan read it (for the fused append)
  int32_t *item_zp;   // [items][4] (slice, first token, end token, 0) of every work item
  int32_t inline_items;  // 1: the split and combine kernels derive the items from lens
  float *part;        // [items][G][4 + d] (max, sum, 0, 0, o) partials
  // Fused append (kv_append_decode_attn_logn), null for plain decode: the token k_new, v_new
  // ([num_slices][d]) each slice appends before it attends.  The split kernel reads the rows
  // before it; the combine kernel merges the token as one more partial and then writes it into
  // the cache through K_app, V_app, N_app, lens_app (the same buffers as K, V, N, lens).
  const char *k_new, *v_new;
  char *K_app, *V_app;
  int32_t *N_app, *lens_app;
};

struct AppArgs {
  char *K, *V;
  int32_t *N, *lens;
  const char *k_new, *v_new;
  int32_t *err;
  int64_t num_slices, cap;
  int32_t rowb;
};

// Bytes of the fixed device scratch array behind decode_attn_logn_noalloc (one per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// Hierarchical centroid index (ball tree per slice, heap order over P leaf slots) and the
// selection of the rows decode attention keeps.
constexpr int kPruneMaxLeaves = 65536;  // largest P (the walk keeps a bit per node of a level)

struct IdxArgs {
  const char *K, *q;
  const int32_t *N, *lens;
  int32_t *err;
  float *mu, *rho, *lmax;  // [num_slices][2P][d], [num_slices][2P] x 2
  int32_t *wt;             // [num_slices][2P] degree totals (0 = empty node)
  int32_t *items;          // build: [num_slices * (P / leaf group)][4] (slice, group, length, 0)
  int32_t *nitems;         // build: number of items
  int64_t num_slices, cap;
  int32_t max_len, d, P, B;
  // pruned decode
  int32_t H_q, H_kv, n1, n2;
  float scale_log2, tau_log2;
  int32_t *runs;      // [num_slices][max_runs][2] kept row runs [first, end)
  int32_t *nruns;     // [num_slices]
  int32_t max_runs, tsplit;
  uint8_t *kept_tap;  // [num_slices][P] or null
  int32_t *item_off;  // [num_slices + 1]
  int32_t *item_zp;   // [items][4]
};

// Storage codes of the C ABI (csmkv_dtype).
constexpr int kDtypeBf16 = 0, kDtypeF32 = 1, kDtypeF16 = 2;

// Each returns 0 or a hipError_t value.
int launch_csm(const CsmArgs &args, int dtype, int d, hipStream_t stream);
int launch_decode(const DecArgs &a, int dtype, int d, int G, int64_t max_items, hipStream_t st);
int launch_append(const AppArgs &a, hipStream_t st);
// op 0: build the index over each slice's rows; op 1: take in the row just appended.
int launch_index(const IdxArgs &a, int dtype, int d, int op, hipStream_t st);
// Leaf slots a build workgroup takes for a tree of P leaf slots (the work table of a build holds
// num_slices * P / this entries).
int32_t index_leaf_group(int32_t P);
// Thresholds, walk and runs per slice, then the item table (the decode split and combine kernels
// follow with launch_decode_table).
int launch_prune(const IdxArgs &a, int dtype, int d, int G, hipStream_t st);
// The decode split and combine kernels over an item table already in args (item_off, item_zp).
int launch_decode_table(const DecArgs &a, int dtype, int d, int G, int64_t max_items, hipStream_t st);
int launch_clear(int32_t *word, hipStream_t st);
// Tokens per decode work item for a geometry, and the upper bound on work items (sizes the
// partial buffer).  Both depend only on the slice count and the host-known length bound.
int32_t dec_split_tokens(int64_t num_slices, int32_t max_len);
int64_t dec_max_items(int64_t num_slices, int32_t max_len);
// Device address of this GPU's scratch array (the current device's), looked up once per
// device; 0 or a hipError_t value.
int noalloc_scratch(void **ptr);

}  // namespace csmkv
