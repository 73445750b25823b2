/*
 * csmkv.h -- C ABI of libcsmkv: Chunked Soft Matching (CSM) KV-cache clustering and
 * log-degree decode attention for AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the pages
 *   "Chelsea: Efficient Long-Context LLM Inference via KV Cache Clustering" (xllm-io paper
 *   review), section 三 技术架构 (核心公式, Algorithm 1, 分块软匹配算法, 定理 6.1), and
 *   "CentroidKV: Efficient Long-Context LLM Inference via KV Cache Clustering" (gist.science),
 *   技术摘要 / 方法论 (推理流水线, 分块软匹配 (CSM), 聚合).
 *
 * Conventions for every entry point
 *   - Pointers to cache data, degrees, lengths, queries, outputs and workspace are DEVICE
 *     pointers owned by the caller.  The library never allocates, frees or keeps them.
 *   - `stream` is the caller's hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; nothing is read back unless the entry point says so.
 *   - Arguments are validated on the host before anything is enqueued.  A negative return
 *     value means nothing was enqueued and no buffer was touched.
 *   - Cache layout: a "slice" is one (batch, layer, kv-head) sequence.  Slices are ordered
 *     slice = group * H_kv + kv_head with group = batch_index * layers + layer.
 *       K, V : [num_slices][cap][d] in `dtype`, token-major, d contiguous
 *       N    : [num_slices][cap] int32, the degree (tokens a row stands for)
 *       lens : [num_slices] int32, the current length s of each slice
 *     K and V must be 16-byte aligned.  Rows at or beyond lens[] are ignored.
 *   - Device-side errors (a lens[] entry above max_len or cap) are reported through an
 *     int32 error word in device memory, read with csmkv_read_error().  The affected
 *     slice is left unchanged (compress, append) or produces zeros (attention).  An in-place
 *     round also sets it if a workgroup's wait for another chunk of its slice does not end
 *     within about a second (the output of that slice is then incomplete); the waits end by
 *     construction, so this only turns a fault that would hang the launch into an error.  The word
 *     is sticky: kernels only ever set it (to CSMKV_EDEVICE), never clear it, so a loop or a
 *     graph replay of many calls reports an error from any of them.  It must hold 0 before
 *     the first call (allocate the workspace zeroed, or call csmkv_clear_error) and is
 *     cleared only by csmkv_clear_error.
 *   - Workspaces: apart from that first int32 (the error word), any prior contents.
 *   - Calls that share a workspace must not overlap in time (use one stream).
 */
#ifndef CSMKV_H
#define CSMKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define CSMKV_API __attribute__((visibility("default")))
#else
#define CSMKV_API
#endif

typedef enum {
  CSMKV_OK = 0,
  CSMKV_EINVAL = -1,        /* argument out of range or required pointer NULL */
  CSMKV_EDTYPE = -2,        /* unknown dtype code */
  CSMKV_EUNSUPPORTED = -3,  /* shape outside what the kernels are built for */
  CSMKV_EWORKSPACE = -4,    /* workspace NULL, misaligned or smaller than required */
  CSMKV_EHIP = -5,          /* a HIP runtime call or kernel launch failed */
  CSMKV_EDEVICE = -6        /* csmkv_read_error: a kernel flagged a bad lens[] entry (or a
                               round's in-place wait that did not end) */
} csmkv_status;

/* Storage formats of K, V (and q).  bf16 is the format the pages use; fp16 (IEEE binary16)
 * and fp32 are supported as well.  Similarities are decided in fp32 in every format and
 * merged centroids are stored rounded to nearest, ties to even. */
typedef enum { CSMKV_BF16 = 0, CSMKV_F32 = 1, CSMKV_F16 = 2 } csmkv_dtype;

typedef struct {
  int64_t num_slices; /* number of (batch, layer, kv-head) slices, >= 0 */
  int64_t cap;        /* rows allocated per slice, >= 1 */
  int32_t d;          /* head dimension: 64 or 128 (other values: CSMKV_EUNSUPPORTED) */
  int32_t dtype;      /* csmkv_dtype of K, V (and q) */
  int32_t max_len;    /* host-known bound on the lens[] entries a call reads, 0 <= max_len
                         <= cap; sizes the launch grids (entries above it are device
                         errors).  In-place rounds exempt outlier slices and
                         csm_compress_triggered slices below their threshold: those are not
                         read, so a bound on the other slices suffices */
} csmkv_cache;

/* Human-readable name of a status code (static string). */
CSMKV_API const char *csmkv_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
CSMKV_API int csmkv_version(void);

/* Bytes of workspace csm_compress / csm_compress_into / csm_compress_debug /
 * csm_compress_triggered need for this
 * cache geometry and these n1, n2, c.  0 if the arguments are invalid. */
CSMKV_API size_t csm_compress_workspace_bytes(const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c);

/*
 * csm_compress -- one CSM round over every slice, in place.
 *   Chelsea review, section 三, 分块软匹配算法 steps 1-4 and Algorithm 1
 *   (K, V, N, s = Chelsea(K, V, N, s, n1, n2, r, c)); CentroidKV page, 分块软匹配 (CSM)
 *   and 聚合.
 * Per slice of length s (slices with outlier_mask[z] != 0 are not read or written):
 *   keep rows [0, n1) and the last n2 rows; split the middle [n1, s-n2) into chunks of c
 *   rows from n1 (the last may be shorter, length L); in each chunk A = even offsets,
 *   B = odd offsets; every A row takes the B row of highest key cosine similarity (lowest
 *   B index on ties); the A rows are ranked by that similarity (descending, lower A index
 *   first on ties) and the first m = floor(r*L/2 + 1e-9) merge into their targets (fp64;
 *   the guard keeps an r*L/2 meant to be whole from rounding below it; m = 0 when L < 2):
 *   k_b <- (N_b k_b + sum N_a k_a) / (N_b + sum N_a), same for v, N_b <- N_b + sum N_a,
 *   accumulated in fp32 in ascending A order and stored with round-to-nearest-even;
 *   merged A rows are removed and the slice is compacted in its original order;
 *   lens[z] becomes s - sum(m).  Similarities are decided in fp32 (bf16 products are
 *   exact, sums rounded in fp32).
 * Arguments: n1, n2 >= 0; 2 <= c <= 512 (c > 256 needs bf16 or fp16 storage: the
 *   similarity tile grows to 256 x 256 and the key tile to c * d * 2 bytes of LDS);
 *   0 <= r <= 1 (not NaN); outlier_mask is a device
 *   [num_slices] uint8 array or NULL (no outliers); workspace: device memory of at least
 *   csm_compress_workspace_bytes() bytes, 256-byte aligned.  Its first int32 is the sticky
 *   error word.
 * Returns CSMKV_OK or a negative csmkv_status.
 */
CSMKV_API int csm_compress(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                 int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * csm_compress_into -- the same round, reading one cache and writing another
 * (out of place).  Outlier slices and the protected rows are copied unchanged.
 * src and dst must agree on num_slices, d and dtype; dst->cap must hold every output
 * (a slice whose output would exceed dst->cap is a device error and is not written).
 * The source buffers are not modified.  Input and output buffers must not overlap.
 */
CSMKV_API int csm_compress_into(const void *K_in, const void *V_in, const int32_t *N_in,
                      const int32_t *lens_in, const csmkv_cache *src,
                      void *K_out, void *V_out, int32_t *N_out, int32_t *lens_out,
                      const csmkv_cache *dst,
                      int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * csm_compress_debug -- csm_compress (in place) that also records its decisions.
 * Not for timed runs.  Any tap may be NULL.
 *   best_b   : [num_slices][units][W] int32, per chunk the matched B index of each A
 *              row (-1 where the row does not exist); units = csm_compress_units();
 *              W = 128 for c <= 256, 256 for larger c.
 *   selected : same shape, uint8, 1 where the A row was merged.
 *   src_pos  : [num_slices][cap] int32, for each output row < new lens the input row it
 *              came from (entries at or beyond the new length are not written).
 */
CSMKV_API int csm_compress_debug(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                       int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                       void *workspace, size_t workspace_bytes, void *stream,
                       int32_t *best_b, uint8_t *selected, int32_t *src_pos);

/*
 * csm_compress_triggered -- csm_compress (in place) with Algorithm 1's trigger and r
 * schedule decided on the device, so that decode steps and their rounds can be enqueued
 * (or captured in a graph) without reading lengths back.
 *   Chelsea review, section 三, Algorithm 1: after an append, cluster when s >= B + g;
 *   CentroidKV page, 渐进式调度: r annealed linearly over the rounds.
 * Per slice z: the round runs only when outlier_mask[z] == 0 and lens[z] >= threshold[z]
 *   (give ceil(B + g): for an integer length, s >= B + g exactly when s >= ceil(B + g));
 *   it then uses r = max(r_init - j * r_delta, r_min), with j = round_index[z] and the
 *   product and difference each rounded once in fp64, and increments round_index[z].
 *   A slice that does not run (or is in error) is left as it is, round_index included.
 *   The round itself is csm_compress's.
 * Arguments: threshold [num_slices] int32 and round_index [num_slices] int32 are device
 *   arrays owned by the caller (round_index is updated in place: it is the schedule state,
 *   start it at the number of rounds already run, e.g. 0 or the prefill round count);
 *   0 <= r_min <= r_init <= 1, r_delta >= 0, none NaN; cache->max_len bounds the length of
 *   every slice that runs (a running slice above it is a device error and is left as it is;
 *   slices that do not run are only checked against cap); the rest as csm_compress.
 * Returns CSMKV_OK or a negative csmkv_status.
 */
CSMKV_API int csm_compress_triggered(void *K, void *V, int32_t *N, int32_t *lens,
                           const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c,
                           const int32_t *threshold, int32_t *round_index, double r_init,
                           double r_delta, double r_min, const uint8_t *outlier_mask,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Chunk units per slice the compress launch uses for this geometry (the leading dimension
 * of the debug taps, which hold one entry block per unit).  0 if invalid. */
CSMKV_API int64_t csm_compress_units(const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c);

/* Bytes of workspace decode_attn_logn needs.  0 if the arguments are invalid. */
CSMKV_API size_t decode_attn_logn_workspace_bytes(const csmkv_cache *cache, int32_t H_q, int32_t H_kv);

/*
 * decode_attn_logn -- grouped-query decode attention over a clustered cache:
 *   O = Softmax(q K^T / sqrt(d) + log N) V
 *   (Chelsea review, section 三, 核心公式: attention with cluster degrees; Algorithm 1
 *   decode output).
 * q : [groups][H_q][d] in the cache dtype, groups = num_slices / H_kv; query head h of
 *   group g reads slice g * H_kv + h / (H_q / H_kv).
 * O : [groups][H_q][d] fp32 (written for every head; an empty slice gives zeros).
 * Arithmetic in fp32 (exp/log in base 2 with the log2(e) factor folded into the scale).  bf16
 * and fp16 caches take q.k and P.V on matrix cores: the q.k products are exact and summed in
 * fp32; P enters P.V as two terms of the storage type (hi + lo, fp16 on a 2^14-scaled P), about
 * 2^-17 (bf16) or 2^-22 (fp16) relative, summed in fp32; the softmax denominator is summed in
 * fp32 from P itself.
 * H_kv >= 1, H_q a multiple of H_kv with H_q / H_kv in {1, 2, 4, 8};
 * num_slices a multiple of H_kv.  Workspace as for csm_compress (first int32 = sticky error
 * word).
 */
CSMKV_API int decode_attn_logn(const void *q, const void *K, const void *V, const int32_t *N,
                     const int32_t *lens, const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                     float *O, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_append_decode_attn_logn -- one decode step of Algorithm 1 in one call: every slice appends
 * the token (k_new, v_new) with degree 1 (as kv_append) and then attends over its rows, the new
 * one included (as decode_attn_logn).
 *   Chelsea review, section 三, Algorithm 1 (K = [K, k], V = [V, v], N = [N, 1], s = s + 1, then
 *   O = Softmax(q K^T / sqrt(d) + log N) V; 核心公式).
 * The attention kernels read the rows that were there before the call; the token enters the
 * last merge of the per-item partials as one more partial, and is then written into the cache
 * (K[s], V[s], N[s] = 1, lens[z] = s + 1).  The output equals that of kv_append followed by
 * decode_attn_logn up to the order of the fp32 sums.  A slice whose length is negative or equal
 * to cap is not appended and sets the error word (its attention then covers its current rows);
 * the length attended over (after the append) must lie within cache->max_len, else the error word
 * is set and that slice's output is zeros (as the two separate calls would give).
 * k_new, v_new : [num_slices][d] in the cache dtype, 16-byte aligned, not NULL.  Other arguments,
 *   layout, workspace (decode_attn_logn_workspace_bytes) and status codes as decode_attn_logn.
 */
CSMKV_API int kv_append_decode_attn_logn(const void *q, void *K, void *V, int32_t *N,
                                         int32_t *lens, const csmkv_cache *cache, int32_t H_q,
                                         int32_t H_kv, const void *k_new, const void *v_new,
                                         float *O, void *workspace, size_t workspace_bytes,
                                         void *stream);

/* Size of the fixed device scratch array decode_attn_logn_noalloc works in (per GPU). */
#define CSMKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * decode_attn_logn_noalloc -- decode_attn_logn for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid allocation.
 * Same computation, same kernels and bit-identical output; the workspace is replaced by a fixed
 * scratch array inside the library (CSMKV_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends), so this call allocates and frees nothing.  Its first call on a device (with that
 * device current) looks up that device's array; later calls only launch kernels.
 * error_word : device int32 owned by the caller (4-byte aligned, not NULL): the sticky error
 *   word of the call (see the conventions above).
 * Geometries whose decode_attn_logn_workspace_bytes() exceed CSMKV_DECODE_NOALLOC_SCRATCH_BYTES
 *   are rejected with CSMKV_EWORKSPACE before anything is enqueued (e.g. 256 slices of up to
 *   64K tokens at G = 4 need about 18 MB; 8192 slices of 32K tokens at G = 1 do not fit).
 * Every call on one GPU uses that GPU's single array: calls that may overlap in time on one GPU
 * (different streams without ordering) race on it and must not be made.  The array keeps the
 * last call's contents; nothing in it needs to start at zero.
 * Other arguments, layout and status codes as decode_attn_logn.
 */
CSMKV_API int decode_attn_logn_noalloc(const void *q, const void *K, const void *V,
                                       const int32_t *N, const int32_t *lens,
                                       const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                                       float *O, int32_t *error_word, void *stream);

/*
 * kv_append -- Algorithm 1 decode update for every slice (Chelsea review, section 三,
 * Algorithm 1: K = [K, k], V = [V, v], N = [N, 1], s = s + 1).
 * k_new, v_new : [num_slices][d] in the cache dtype.  A slice whose lens is negative or
 * already equal to cap is not written and sets *error_word (device int32, may be NULL)
 * to CSMKV_EDEVICE.  max_len is not used by this call.
 */
CSMKV_API int kv_append(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
              const void *k_new, const void *v_new, int32_t *error_word, void *stream);

/* ---------------------------------------------------------------- CPU-offloaded clustering
 * CentroidKV page, 它做不到的事（局限性） → 仍留在 GPU 上 and 技术摘要 → 作者注明的局限性: the
 * grouping could run on the CPU with only its result sent to the GPU.  These two entry points do
 * that: a CSM round over a cache held in HOST memory, on the host's cores, and an asynchronous
 * copy of the compacted rows into the device cache.
 */

/* Vector unit csm_compress_host uses on this CPU (chosen at run time). */
#define CSMKV_HOST_ISA_SCALAR 0
#define CSMKV_HOST_ISA_AVX2 1   /* AVX2 + FMA */
#define CSMKV_HOST_ISA_AVX512 2 /* AVX-512F */
CSMKV_API int csm_host_isa(void);

/*
 * csm_compress_host -- csm_compress's round (same arguments, rules and readings) on a cache in
 * HOST memory, in place, on num_threads host threads (0 = one per hardware thread), one slice per
 * thread at a time.  K, V, N, lens and outlier_mask (NULL = none) are host pointers in the device
 * layout.  Similarities in fp32 (exact bf16 / fp16 products), merges accumulated in fp32 and
 * rounded to nearest even, like the device round; results agree with it up to near-ties.
 * Optional host taps as csm_compress_debug (best_b and selected both or neither; units from
 * cache->max_len, which must then bound every slice that runs; src_pos [num_slices][cap]).
 * Every lens[] entry is checked against cap first: CSMKV_EINVAL and nothing changed if one is
 * out of range.  Blocks until done.  Returns CSMKV_OK or a negative csmkv_status.
 */
CSMKV_API int csm_compress_host(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                                int32_t n1, int32_t n2, int32_t c, double r,
                                const uint8_t *outlier_mask, int32_t num_threads, int32_t *best_b,
                                uint8_t *selected, int32_t *src_pos);

/*
 * csm_upload_rows -- enqueue on `stream` the copy of a host cache's rows [row_begin, lens_host[z])
 * (K, V, N) and lens_host[z] into the device cache, for every slice z with outlier_mask[z] == 0
 * (outlier_mask: host pointer or NULL = every slice).  After csm_compress_host the rows from n1
 * on are the ones a round changed, so row_begin = n1 sends only the round's result.  Consecutive
 * slices go as one strided copy each for K, V, N and lens (rows between a slice's length and its
 * group's longest may be copied too; they lie past its length).  Host buffers must stay
 * unchanged until the stream has run the copies, and should be pinned (hipHostMalloc) for the
 * copies to be asynchronous.  Both caches share `cache`'s geometry.  Returns CSMKV_OK,
 * CSMKV_EINVAL (NULL pointer, row_begin < 0, a lens_host entry out of [0, cap]) with nothing
 * enqueued, or CSMKV_EHIP.
 */
CSMKV_API int csm_upload_rows(const void *K_host, const void *V_host, const int32_t *N_host,
                              const int32_t *lens_host, void *K, void *V, int32_t *N,
                              int32_t *lens, const csmkv_cache *cache, int32_t row_begin,
                              const uint8_t *outlier_mask, void *stream);

/* ---------------------------------------------------------------- hierarchical centroid index
 * LycheeCluster page, 方法论 §2 层次 KV 索引 and §3 流式懒更新: block centroids in a binary tree
 * whose distances obey the triangle inequality, walked by the query to drop whole subtrees, and
 * refreshed lazily as tokens are appended.  Here, over the cache CSM leaves: per slice a ball tree
 * over blocks of block_rows consecutive rows (a leaf: centre = degree-weighted mean of its keys,
 * radius = farthest key; an inner node: centre = degree-weighted mean of its children's centres,
 * radius covering both child balls), in heap order over P leaf slots, P = the power of two that
 * holds cap / block_rows blocks (at most 65536).  block_rows: 16, 32, 64, 128 or 256.
 * Index memory (device, caller-owned, 256-byte aligned): csm_index_bytes() bytes, laid out as
 * centres [num_slices][2P][d] fp32, radii, largest log2 degree and degree totals [num_slices][2P],
 * then a work table the build fills and reads (one 16-byte entry per group of eight leaf slots).
 */
CSMKV_API size_t csm_index_bytes(const csmkv_cache *cache, int32_t block_rows);

/* Build every slice's tree over its rows [0, lens[z]) (after a CSM round, or any change of the
 * rows).  error_word: device int32 (sticky), set for a lens[] entry above max_len or cap (that
 * slice's tree is left empty).  Returns CSMKV_OK or a negative csmkv_status. */
CSMKV_API int csm_index_build(const void *K, const int32_t *N, const int32_t *lens,
                              const csmkv_cache *cache, int32_t block_rows, void *index,
                              size_t index_bytes, int32_t *error_word, void *stream);

/* Take in the row lens[z] - 1 just appended to every slice (after kv_append), lazily: the row
 * joins its leaf (or opens a new one centred on it); the leaf's and every ancestor's radius grow
 * to cover it; centres move only at the next build.  Bounds stay valid. */
CSMKV_API int csm_index_append(const void *K, const int32_t *N, const int32_t *lens,
                               const csmkv_cache *cache, int32_t block_rows, void *index,
                               size_t index_bytes, int32_t *error_word, void *stream);

/* Workspace bytes of decode_attn_logn_pruned (first int32: the sticky error word). */
CSMKV_API size_t decode_attn_logn_pruned_workspace_bytes(const csmkv_cache *cache, int32_t H_q,
                                                         int32_t H_kv, int32_t block_rows);

/*
 * decode_attn_logn_pruned -- decode_attn_logn over the rows the index keeps.  Per slice (its G
 * query heads together): every key k in a node's ball satisfies q.k <= q.mu + |q| rho, so
 * U = (q.mu + |q| rho) log2(e) / sqrt(d) + max log2 N bounds the base-2 logit of all its rows.
 * m_low = the largest exact logit among the protected rows (the first n1, the last n2) and the
 * first row of every block.  The tree is walked from the root, a node's children visited only if
 * U >= m_low - tau log2(e) for one of the G heads; blocks that pass, and blocks holding a
 * protected row, are kept, and O is the log-N attention over their rows.  tau = +inf keeps every
 * block.  A dropped row weighs at most e^-tau of the largest, which is always kept.
 * kept: optional device [num_slices][P] uint8 tap (1 = block kept).  Other arguments as
 * decode_attn_logn; the index must describe the current rows (built, and appended to after each
 * kv_append).
 */
CSMKV_API int decode_attn_logn_pruned(const void *q, const void *K, const void *V, const int32_t *N,
                                      const int32_t *lens, const csmkv_cache *cache, int32_t H_q,
                                      int32_t H_kv, int32_t n1, int32_t n2, int32_t block_rows,
                                      const void *index, size_t index_bytes, double tau, float *O,
                                      uint8_t *kept, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Synchronise `stream` and return CSMKV_OK if the device error word is 0, CSMKV_EDEVICE if
 * a kernel set it, or CSMKV_EHIP if the copy failed.  error_word is the first int32 of a
 * workspace or the word given to kv_append.  The word is not changed. */
CSMKV_API int csmkv_read_error(const int32_t *error_word, void *stream);

/* Enqueue on `stream` a reset of a device error word to 0 (a one-thread kernel, so it can be
 * captured in a graph).  error_word: device int32, 4-byte aligned.  Returns CSMKV_OK,
 * CSMKV_EINVAL (NULL or misaligned) or CSMKV_EHIP. */
CSMKV_API int csmkv_clear_error(int32_t *error_word, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSMKV_H */
