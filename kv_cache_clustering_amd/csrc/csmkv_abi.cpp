// C ABI of libcsmkv (declared in include/csmkv.h): host-side validation, workspace layout
// and launches on the caller's stream.  No entry point allocates or frees memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "csmkv.h"

#include "kernel_args.hpp"

namespace {

constexpr int64_t kMaxCap = int64_t(1) << 24;  // degrees and row indices stay exact in fp32 / int32
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int32_t dtype) { return dtype == CSMKV_F32 ? 4 : 2; }

int check_cache(const csmkv_cache *c) {
  if (c == nullptr) return CSMKV_EINVAL;
  if (c->dtype != CSMKV_BF16 && c->dtype != CSMKV_F32 && c->dtype != CSMKV_F16)
    return CSMKV_EDTYPE;
  if (c->num_slices < 0 || c->cap < 1 || c->d < 1) return CSMKV_EINVAL;
  if (c->max_len < 0 || (int64_t)c->max_len > c->cap) return CSMKV_EINVAL;
  if (c->d != 64 && c->d != 128) return CSMKV_EUNSUPPORTED;
  if (c->cap > kMaxCap) return CSMKV_EUNSUPPORTED;
  return CSMKV_OK;
}

int64_t units_per_slice(int32_t max_len, int32_t n1, int32_t n2, int32_t c) {
  const int64_t M = (int64_t)max_len - n1 - n2;
  const int64_t nch = M >= 2 ? (M + c - 1) / c : 0;
  return nch + 1;  // chunks + the tail unit
}

int check_csm_params(int32_t n1, int32_t n2, int32_t c, double r) {
  if (n1 < 0 || n2 < 0) return CSMKV_EINVAL;
  if (c < 2) return CSMKV_EINVAL;
  if (c > 512) return CSMKV_EUNSUPPORTED;
  if (!(r >= 0.0 && r <= 1.0)) return CSMKV_EINVAL;  // also rejects NaN
  return CSMKV_OK;
}

struct CsmLayout {
  size_t ticket, s_in, s_out, s_r, flags, total;
};

CsmLayout csm_layout(int64_t S, int64_t units) {
  CsmLayout L;
  L.ticket = kAlign;
  L.s_in = L.ticket + align_up((size_t)S * 4);
  L.s_out = L.s_in + align_up((size_t)S * 4);
  L.s_r = L.s_out + align_up((size_t)S * 4);
  L.flags = L.s_r + align_up((size_t)S * 8);
  L.total = L.flags + align_up((size_t)(S * units) * 4);
  return L;
}

int csm_common(const void *K_in, const void *V_in, const int32_t *N_in, const int32_t *lens_in,
               const csmkv_cache *src, void *K_out, void *V_out, int32_t *N_out,
               int32_t *lens_out, const csmkv_cache *dst, int32_t n1, int32_t n2, int32_t c,
               double r, const uint8_t *mask, void *ws, size_t ws_bytes, void *stream,
               int in_place, int32_t *tap_best, uint8_t *tap_sel, int32_t *tap_src,
               const int32_t *thr = nullptr, int32_t *round_idx = nullptr, double r_init = 0.0,
               double r_delta = 0.0, double r_min = 0.0) {
  int rc = check_cache(src);
  if (rc) return rc;
  rc = check_cache(dst);
  if (rc) return rc;
  if (src->num_slices != dst->num_slices || src->d != dst->d || src->dtype != dst->dtype)
    return CSMKV_EINVAL;
  rc = check_csm_params(n1, n2, c, r);
  if (rc) return rc;
  if (c > 256 && src->dtype == CSMKV_F32) return CSMKV_EUNSUPPORTED;  // no fp32 512-row tile
  if (!K_in || !V_in || !N_in || !lens_in || !K_out || !V_out || !N_out || !lens_out)
    return CSMKV_EINVAL;
  if (!aligned(K_in, 16) || !aligned(V_in, 16) || !aligned(K_out, 16) || !aligned(V_out, 16))
    return CSMKV_EINVAL;
  if (tap_sel != nullptr && tap_best == nullptr) return CSMKV_EINVAL;
  if (tap_best != nullptr && tap_sel == nullptr) return CSMKV_EINVAL;
  const int64_t S = src->num_slices;
  const int64_t units = units_per_slice(src->max_len, n1, n2, c);
  if (S * units > (int64_t)INT32_MAX) return CSMKV_EUNSUPPORTED;
  const CsmLayout lay = csm_layout(S, units);
  if (ws == nullptr || !aligned(ws, kAlign) || ws_bytes < lay.total) return CSMKV_EWORKSPACE;
  char *w = static_cast<char *>(ws);
  csmkv::CsmArgs a;
  a.Kin = static_cast<const char *>(K_in);
  a.Vin = static_cast<const char *>(V_in);
  a.Nin = N_in;
  a.Kout = static_cast<char *>(K_out);
  a.Vout = static_cast<char *>(V_out);
  a.Nout = N_out;
  a.lens_out = lens_out;
  a.lens_in = lens_in;
  a.mask = mask;
  a.num_slices = S;
  a.cap_in = src->cap;
  a.cap_out = dst->cap;
  a.max_len = src->max_len;
  a.n1 = n1;
  a.n2 = n2;
  a.c = c;
  a.units = (int32_t)units;
  a.in_place = in_place;
  a.r = r;
  a.thr = thr;
  a.round_idx = round_idx;
  a.r_init = r_init;
  a.r_delta = r_delta;
  a.r_min = r_min;
  a.err = reinterpret_cast<int32_t *>(w);
  a.ticket = reinterpret_cast<uint32_t *>(w + lay.ticket);
  a.s_in = reinterpret_cast<int32_t *>(w + lay.s_in);
  a.s_out = reinterpret_cast<int32_t *>(w + lay.s_out);
  a.s_r = reinterpret_cast<double *>(w + lay.s_r);
  a.flags = reinterpret_cast<int32_t *>(w + lay.flags);
  a.tap_best = tap_best;
  a.tap_sel = tap_sel;
  a.tap_src = tap_src;
  if (S == 0) return CSMKV_OK;
  const int e = csmkv::launch_csm(a, src->dtype, src->d, static_cast<hipStream_t>(stream));
  return e ? CSMKV_EHIP : CSMKV_OK;
}

struct DecLayout {
  size_t item_off, s_in, item_zp, part, total;
};

DecLayout dec_layout(const csmkv_cache *c, int G) {
  DecLayout L;
  const int64_t items = csmkv::dec_max_items(c->num_slices, c->max_len);
  L.item_off = kAlign;
  L.s_in = L.item_off + align_up((size_t)(c->num_slices + 1) * 4);
  L.item_zp = L.s_in + align_up((size_t)c->num_slices * 4);
  L.part = L.item_zp + align_up((size_t)items * 16);
  L.total = L.part + align_up((size_t)items * G * (4 + c->d) * 4);
  return L;
}

int check_heads(const csmkv_cache *c, int32_t H_q, int32_t H_kv) {
  if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0) return CSMKV_EINVAL;
  if (c->num_slices % H_kv != 0) return CSMKV_EINVAL;
  const int G = H_q / H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return CSMKV_EUNSUPPORTED;
  return CSMKV_OK;
}

}  // namespace

extern "C" {

const char *csmkv_status_string(int status) {
  switch (status) {
    case CSMKV_OK: return "CSMKV_OK";
    case CSMKV_EINVAL: return "CSMKV_EINVAL: argument out of range or required pointer NULL";
    case CSMKV_EDTYPE: return "CSMKV_EDTYPE: unknown dtype";
    case CSMKV_EUNSUPPORTED: return "CSMKV_EUNSUPPORTED: shape outside the built kernels";
    case CSMKV_EWORKSPACE: return "CSMKV_EWORKSPACE: workspace missing, misaligned or too small";
    case CSMKV_EHIP: return "CSMKV_EHIP: HIP runtime call or kernel launch failed";
    case CSMKV_EDEVICE: return "CSMKV_EDEVICE: a kernel flagged an invalid lens[] entry";
    default: return "unknown csmkv status";
  }
}

int csmkv_version(void) { return 106; }

size_t csm_compress_workspace_bytes(const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c) {
  if (check_cache(cache) || n1 < 0 || n2 < 0 || c < 2 || c > 512) return 0;
  const int64_t units = units_per_slice(cache->max_len, n1, n2, c);
  return csm_layout(cache->num_slices, units).total;
}

int csm_compress_triggered(void *K, void *V, int32_t *N, int32_t *lens,
                           const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c,
                           const int32_t *threshold, int32_t *round_index, double r_init,
                           double r_delta, double r_min, const uint8_t *outlier_mask,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (threshold == nullptr || round_index == nullptr) return CSMKV_EINVAL;
  if (!(r_delta >= 0.0) || !(r_min >= 0.0 && r_min <= 1.0) || !(r_init >= r_min && r_init <= 1.0))
    return CSMKV_EINVAL;  // also rejects NaN; every annealed r then lies in [r_min, r_init]
  return csm_common(K, V, N, lens, cache, K, V, N, lens, cache, n1, n2, c, r_init, outlier_mask,
                    workspace, workspace_bytes, stream, 1, nullptr, nullptr, nullptr, threshold,
                    round_index, r_init, r_delta, r_min);
}

int64_t csm_compress_units(const csmkv_cache *cache, int32_t n1, int32_t n2, int32_t c) {
  if (check_cache(cache) || n1 < 0 || n2 < 0 || c < 2 || c > 512) return 0;
  return units_per_slice(cache->max_len, n1, n2, c);
}

int csm_compress(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                 int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                 void *workspace, size_t workspace_bytes, void *stream) {
  return csm_common(K, V, N, lens, cache, K, V, N, lens, cache, n1, n2, c, r, outlier_mask,
                    workspace, workspace_bytes, stream, 1, nullptr, nullptr, nullptr);
}

int csm_compress_debug(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
                       int32_t n1, int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                       void *workspace, size_t workspace_bytes, void *stream, int32_t *best_b,
                       uint8_t *selected, int32_t *src_pos) {
  return csm_common(K, V, N, lens, cache, K, V, N, lens, cache, n1, n2, c, r, outlier_mask,
                    workspace, workspace_bytes, stream, 1, best_b, selected, src_pos);
}

int csm_compress_into(const void *K_in, const void *V_in, const int32_t *N_in,
                      const int32_t *lens_in, const csmkv_cache *src, void *K_out, void *V_out,
                      int32_t *N_out, int32_t *lens_out, const csmkv_cache *dst, int32_t n1,
                      int32_t n2, int32_t c, double r, const uint8_t *outlier_mask,
                      void *workspace, size_t workspace_bytes, void *stream) {
  if (K_in == K_out || V_in == V_out || N_in == N_out || lens_in == lens_out) return CSMKV_EINVAL;
  return csm_common(K_in, V_in, N_in, lens_in, src, K_out, V_out, N_out, lens_out, dst, n1, n2, c,
                    r, outlier_mask, workspace, workspace_bytes, stream, 0, nullptr, nullptr,
                    nullptr);
}

size_t decode_attn_logn_workspace_bytes(const csmkv_cache *cache, int32_t H_q, int32_t H_kv) {
  if (check_cache(cache) || check_heads(cache, H_q, H_kv)) return 0;
  return dec_layout(cache, H_q / H_kv).total;
}

namespace {

// decode_attn_logn, and with k_new / v_new the fused append of kv_append_decode_attn_logn.
int decode_common(const void *q, const void *K, const void *V, const int32_t *N,
                  const int32_t *lens, const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                  float *O, void *workspace, size_t workspace_bytes, void *stream,
                  const void *k_new, const void *v_new) {
  int rc = check_cache(cache);
  if (rc) return rc;
  rc = check_heads(cache, H_q, H_kv);
  if (rc) return rc;
  if (!q || !K || !V || !N || !lens || !O) return CSMKV_EINVAL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16)) return CSMKV_EINVAL;
  const bool fuse = k_new != nullptr || v_new != nullptr;
  if (fuse && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
    return CSMKV_EINVAL;
  const int G = H_q / H_kv;
  const DecLayout lay = dec_layout(cache, G);
  if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < lay.total)
    return CSMKV_EWORKSPACE;
  const int64_t items = csmkv::dec_max_items(cache->num_slices, cache->max_len);
  if (items > (int64_t)INT32_MAX / 2) return CSMKV_EUNSUPPORTED;
  if (cache->num_slices == 0) return CSMKV_OK;
  char *w = static_cast<char *>(workspace);
  csmkv::DecArgs a = {};
  a.q = static_cast<const char *>(q);
  a.K = static_cast<const char *>(K);
  a.V = static_cast<const char *>(V);
  a.N = N;
  a.lens = lens;
  a.O = O;
  a.num_slices = cache->num_slices;
  a.cap = cache->cap;
  a.max_len = cache->max_len;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.tsplit = csmkv::dec_split_tokens(cache->num_slices, cache->max_len);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cache->d));
  a.err = reinterpret_cast<int32_t *>(w);
  a.item_off = reinterpret_cast<int32_t *>(w + lay.item_off);
  a.s_in = reinterpret_cast<int32_t *>(w + lay.s_in);
  a.item_zp = reinterpret_cast<int32_t *>(w + lay.item_zp);
  a.part = reinterpret_cast<float *>(w + lay.part);
  if (fuse) {  // the caller passed writable cache buffers (kv_append_decode_attn_logn)
    a.k_new = static_cast<const char *>(k_new);
    a.v_new = static_cast<const char *>(v_new);
    a.K_app = const_cast<char *>(a.K);
    a.V_app = const_cast<char *>(a.V);
    a.N_app = const_cast<int32_t *>(N);
    a.lens_app = const_cast<int32_t *>(lens);
  }
  const int e = csmkv::launch_decode(a, cache->dtype, cache->d, G, items,
                                     static_cast<hipStream_t>(stream));
  return e ? CSMKV_EHIP : CSMKV_OK;
}

}  // namespace

int decode_attn_logn(const void *q, const void *K, const void *V, const int32_t *N,
                     const int32_t *lens, const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                     float *O, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_common(q, K, V, N, lens, cache, H_q, H_kv, O, workspace, workspace_bytes, stream,
                       nullptr, nullptr);
}

int kv_append_decode_attn_logn(const void *q, void *K, void *V, int32_t *N, int32_t *lens,
                               const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                               const void *k_new, const void *v_new, float *O, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (!k_new || !v_new) return CSMKV_EINVAL;
  return decode_common(q, K, V, N, lens, cache, H_q, H_kv, O, workspace, workspace_bytes, stream,
                       k_new, v_new);
}

int decode_attn_logn_noalloc(const void *q, const void *K, const void *V, const int32_t *N,
                             const int32_t *lens, const csmkv_cache *cache, int32_t H_q,
                             int32_t H_kv, float *O, int32_t *error_word, void *stream) {
  static_assert(csmkv::kNoAllocScratchBytes == CSMKV_DECODE_NOALLOC_SCRATCH_BYTES,
                "scratch size in the header and the library agree");
  int rc = check_cache(cache);
  if (rc) return rc;
  rc = check_heads(cache, H_q, H_kv);
  if (rc) return rc;
  if (!q || !K || !V || !N || !lens || !O || !error_word) return CSMKV_EINVAL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(error_word, 4))
    return CSMKV_EINVAL;
  const int G = H_q / H_kv;
  const DecLayout lay = dec_layout(cache, G);
  if (lay.total > CSMKV_DECODE_NOALLOC_SCRATCH_BYTES) return CSMKV_EWORKSPACE;
  const int64_t items = csmkv::dec_max_items(cache->num_slices, cache->max_len);
  if (items > (int64_t)INT32_MAX / 2) return CSMKV_EUNSUPPORTED;
  if (cache->num_slices == 0) return CSMKV_OK;
  void *scr = nullptr;
  if (csmkv::noalloc_scratch(&scr) != 0) return CSMKV_EHIP;
  char *w = static_cast<char *>(scr);
  csmkv::DecArgs a = {};
  a.q = static_cast<const char *>(q);
  a.K = static_cast<const char *>(K);
  a.V = static_cast<const char *>(V);
  a.N = N;
  a.lens = lens;
  a.O = O;
  a.num_slices = cache->num_slices;
  a.cap = cache->cap;
  a.max_len = cache->max_len;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.tsplit = csmkv::dec_split_tokens(cache->num_slices, cache->max_len);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cache->d));
  a.err = error_word;
  a.item_off = reinterpret_cast<int32_t *>(w + lay.item_off);
  a.s_in = reinterpret_cast<int32_t *>(w + lay.s_in);
  a.item_zp = reinterpret_cast<int32_t *>(w + lay.item_zp);
  a.part = reinterpret_cast<float *>(w + lay.part);
  const int e = csmkv::launch_decode(a, cache->dtype, cache->d, G, items,
                                     static_cast<hipStream_t>(stream));
  return e ? CSMKV_EHIP : CSMKV_OK;
}

int kv_append(void *K, void *V, int32_t *N, int32_t *lens, const csmkv_cache *cache,
              const void *k_new, const void *v_new, int32_t *error_word, void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (!K || !V || !N || !lens || !k_new || !v_new) return CSMKV_EINVAL;
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(k_new, 16) || !aligned(v_new, 16))
    return CSMKV_EINVAL;
  if (cache->num_slices * 16 > (int64_t)INT32_MAX * 128) return CSMKV_EUNSUPPORTED;
  csmkv::AppArgs a;
  a.K = static_cast<char *>(K);
  a.V = static_cast<char *>(V);
  a.N = N;
  a.lens = lens;
  a.k_new = static_cast<const char *>(k_new);
  a.v_new = static_cast<const char *>(v_new);
  a.err = error_word;
  a.num_slices = cache->num_slices;
  a.cap = cache->cap;
  a.rowb = cache->d * elem_bytes(cache->dtype);
  const int e = csmkv::launch_append(a, static_cast<hipStream_t>(stream));
  return e ? CSMKV_EHIP : CSMKV_OK;
}

int csm_upload_rows(const void *K_host, const void *V_host, const int32_t *N_host,
                    const int32_t *lens_host, void *K, void *V, int32_t *N, int32_t *lens,
                    const csmkv_cache *cache, int32_t row_begin, const uint8_t *outlier_mask,
                    void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (!K_host || !V_host || !N_host || !lens_host || !K || !V || !N || !lens || row_begin < 0)
    return CSMKV_EINVAL;
  const int64_t S = cache->num_slices, cap = cache->cap;
  for (int64_t z = 0; z < S; ++z)
    if (lens_host[z] < 0 || (int64_t)lens_host[z] > cap) return CSMKV_EINVAL;
  const size_t rowb = (size_t)cache->d * elem_bytes(cache->dtype);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char *Kh = static_cast<const char *>(K_host), *Vh = static_cast<const char *>(V_host);
  char *Kd = static_cast<char *>(K), *Vd = static_cast<char *>(V);
  for (int64_t z0 = 0; z0 < S;) {
    if (outlier_mask && outlier_mask[z0]) {
      ++z0;
      continue;
    }
    int64_t z1 = z0;  // a run of consecutive slices to upload
    int64_t hi = 0;
    while (z1 < S && !(outlier_mask && outlier_mask[z1])) hi = std::max<int64_t>(hi, lens_host[z1++]);
    const size_t run = (size_t)(z1 - z0);
    if (hi > row_begin) {
      const size_t rows = (size_t)(hi - row_begin);
      const size_t off = ((size_t)z0 * cap + row_begin) * rowb, pitch = (size_t)cap * rowb;
      const size_t noff = (size_t)z0 * cap + row_begin, npitch = (size_t)cap * 4;
      if (hipMemcpy2DAsync(Kd + off, pitch, Kh + off, pitch, rows * rowb, run, hipMemcpyHostToDevice, st) != hipSuccess ||
          hipMemcpy2DAsync(Vd + off, pitch, Vh + off, pitch, rows * rowb, run, hipMemcpyHostToDevice, st) != hipSuccess ||
          hipMemcpy2DAsync(N + noff, npitch, N_host + noff, npitch, rows * 4, run, hipMemcpyHostToDevice, st) != hipSuccess)
        return CSMKV_EHIP;
    }
    if (hipMemcpyAsync(lens + z0, lens_host + z0, run * 4, hipMemcpyHostToDevice, st) != hipSuccess)
      return CSMKV_EHIP;
    z0 = z1;
  }
  return CSMKV_OK;
}

// ---------------------------------------------------------------- hierarchical centroid index
namespace {

// Leaf slots of a slice's tree: the smallest power of two holding cap / B blocks; 0 if invalid.
int64_t index_leaf_slots(const csmkv_cache *c, int32_t B) {
  if (B != 16 && B != 32 && B != 64 && B != 128 && B != 256) return 0;
  const int64_t leaves = (c->cap + B - 1) / B;
  int64_t P = 1;
  while (P < leaves) P *= 2;
  return P <= csmkv::kPruneMaxLeaves ? P : 0;
}

struct IdxLayout {
  size_t mu, rho, lmax, wt, items, nitems, total;
};
IdxLayout idx_layout(const csmkv_cache *c, int64_t P) {
  IdxLayout L;
  const size_t nodes = (size_t)c->num_slices * 2 * (size_t)P;
  // the build's work table: one 16-byte entry per leaf group of every slice
  const size_t groups = (size_t)c->num_slices * (size_t)(P / csmkv::index_leaf_group((int32_t)P));
  L.mu = 0;
  L.rho = align_up(nodes * (size_t)c->d * 4);
  L.lmax = L.rho + align_up(nodes * 4);
  L.wt = L.lmax + align_up(nodes * 4);
  L.items = L.wt + align_up(nodes * 4);
  L.nitems = L.items + align_up(groups * 16);
  L.total = L.nitems + kAlign;
  return L;
}

int index_common(const void *K, const int32_t *N, const int32_t *lens, const csmkv_cache *cache,
                 int32_t B, void *index, size_t index_bytes, int32_t *error_word, void *stream,
                 int op) {
  int rc = check_cache(cache);
  if (rc) return rc;
  const int64_t P = index_leaf_slots(cache, B);
  if (P == 0) return CSMKV_EUNSUPPORTED;
  if (!K || !N || !lens || !index || !error_word) return CSMKV_EINVAL;
  if (!aligned(K, 16) || !aligned(index, kAlign) || !aligned(error_word, 4)) return CSMKV_EINVAL;
  // work-table entries are counted in int32
  if (cache->num_slices * (P / csmkv::index_leaf_group((int32_t)P)) > (int64_t)INT32_MAX / 4)
    return CSMKV_EUNSUPPORTED;
  const IdxLayout lay = idx_layout(cache, P);
  if (index_bytes < lay.total) return CSMKV_EWORKSPACE;
  char *x = static_cast<char *>(index);
  csmkv::IdxArgs a = {};
  a.K = static_cast<const char *>(K);
  a.N = N;
  a.lens = lens;
  a.err = error_word;
  a.mu = reinterpret_cast<float *>(x + lay.mu);
  a.rho = reinterpret_cast<float *>(x + lay.rho);
  a.lmax = reinterpret_cast<float *>(x + lay.lmax);
  a.wt = reinterpret_cast<int32_t *>(x + lay.wt);
  a.items = reinterpret_cast<int32_t *>(x + lay.items);
  a.nitems = reinterpret_cast<int32_t *>(x + lay.nitems);
  a.num_slices = cache->num_slices;
  a.cap = cache->cap;
  a.max_len = cache->max_len;
  a.d = cache->d;
  a.P = (int32_t)P;
  a.B = B;
  const int e = csmkv::launch_index(a, cache->dtype, cache->d, op, static_cast<hipStream_t>(stream));
  return e ? CSMKV_EHIP : CSMKV_OK;
}

struct PruneLayout {
  size_t item_off, item_zp, part, runs, nruns, total;
  int64_t items, max_runs;
};
PruneLayout prune_layout(const csmkv_cache *c, int G, int64_t P) {
  PruneLayout L;
  const int32_t ts = csmkv::dec_split_tokens(c->num_slices, c->max_len);
  L.max_runs = P / 2 + 1;
  L.items = c->num_slices * (L.max_runs + (c->max_len + ts - 1) / ts);
  L.item_off = kAlign;
  L.item_zp = L.item_off + align_up((size_t)(c->num_slices + 1) * 4);
  L.part = L.item_zp + align_up((size_t)L.items * 16);
  L.runs = L.part + align_up((size_t)L.items * G * (4 + c->d) * 4);
  L.nruns = L.runs + align_up((size_t)c->num_slices * L.max_runs * 8);
  L.total = L.nruns + align_up((size_t)c->num_slices * 4);
  return L;
}

}  // namespace

size_t csm_index_bytes(const csmkv_cache *cache, int32_t block_rows) {
  if (check_cache(cache)) return 0;
  const int64_t P = index_leaf_slots(cache, block_rows);
  return P ? idx_layout(cache, P).total : 0;
}

int csm_index_build(const void *K, const int32_t *N, const int32_t *lens, const csmkv_cache *cache,
                    int32_t block_rows, void *index, size_t index_bytes, int32_t *error_word,
                    void *stream) {
  return index_common(K, N, lens, cache, block_rows, index, index_bytes, error_word, stream, 0);
}

int csm_index_append(const void *K, const int32_t *N, const int32_t *lens, const csmkv_cache *cache,
                     int32_t block_rows, void *index, size_t index_bytes, int32_t *error_word,
                     void *stream) {
  return index_common(K, N, lens, cache, block_rows, index, index_bytes, error_word, stream, 1);
}

size_t decode_attn_logn_pruned_workspace_bytes(const csmkv_cache *cache, int32_t H_q, int32_t H_kv,
                                               int32_t block_rows) {
  if (check_cache(cache) || check_heads(cache, H_q, H_kv)) return 0;
  const int64_t P = index_leaf_slots(cache, block_rows);
  return P ? prune_layout(cache, H_q / H_kv, P).total : 0;
}

int decode_attn_logn_pruned(const void *q, const void *K, const void *V, const int32_t *N,
                            const int32_t *lens, const csmkv_cache *cache, int32_t H_q,
                            int32_t H_kv, int32_t n1, int32_t n2, int32_t block_rows,
                            const void *index, size_t index_bytes, double tau, float *O,
                            uint8_t *kept, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  rc = check_heads(cache, H_q, H_kv);
  if (rc) return rc;
  const int64_t P = index_leaf_slots(cache, block_rows);
  if (P == 0) return CSMKV_EUNSUPPORTED;
  if (!q || !K || !V || !N || !lens || !O || !index || n1 < 0 || n2 < 0 || !(tau >= 0.0))
    return CSMKV_EINVAL;  // tau may be +inf (nothing dropped); NaN is rejected
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(index, kAlign))
    return CSMKV_EINVAL;
  const IdxLayout il = idx_layout(cache, P);
  if (index_bytes < il.total) return CSMKV_EWORKSPACE;
  const int G = H_q / H_kv;
  const PruneLayout lay = prune_layout(cache, G, P);
  if (workspace == nullptr || !aligned(workspace, kAlign) || workspace_bytes < lay.total)
    return CSMKV_EWORKSPACE;
  if (lay.items > (int64_t)INT32_MAX / 2) return CSMKV_EUNSUPPORTED;
  if (cache->num_slices == 0) return CSMKV_OK;
  char *w = static_cast<char *>(workspace);
  char *x = const_cast<char *>(static_cast<const char *>(index));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cache->d));
  const int32_t ts = csmkv::dec_split_tokens(cache->num_slices, cache->max_len);
  csmkv::IdxArgs a = {};
  a.K = static_cast<const char *>(K);
  a.q = static_cast<const char *>(q);
  a.N = N;
  a.lens = lens;
  a.err = reinterpret_cast<int32_t *>(w);
  a.mu = reinterpret_cast<float *>(x + il.mu);
  a.rho = reinterpret_cast<float *>(x + il.rho);
  a.lmax = reinterpret_cast<float *>(x + il.lmax);
  a.wt = reinterpret_cast<int32_t *>(x + il.wt);
  a.num_slices = cache->num_slices;
  a.cap = cache->cap;
  a.max_len = cache->max_len;
  a.d = cache->d;
  a.P = (int32_t)P;
  a.B = block_rows;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.n1 = n1;
  a.n2 = n2;
  a.scale_log2 = scale_log2;
  a.tau_log2 = std::isinf(tau) ? INFINITY : (float)(tau * 1.4426950408889634);
  a.runs = reinterpret_cast<int32_t *>(w + lay.runs);
  a.nruns = reinterpret_cast<int32_t *>(w + lay.nruns);
  a.max_runs = (int32_t)lay.max_runs;
  a.tsplit = ts;
  a.kept_tap = kept;
  a.item_off = reinterpret_cast<int32_t *>(w + lay.item_off);
  a.item_zp = reinterpret_cast<int32_t *>(w + lay.item_zp);
  int e = csmkv::launch_prune(a, cache->dtype, cache->d, G, st);
  if (e) return CSMKV_EHIP;
  csmkv::DecArgs da = {};
  da.q = static_cast<const char *>(q);
  da.K = static_cast<const char *>(K);
  da.V = static_cast<const char *>(V);
  da.N = N;
  da.lens = lens;
  da.O = O;
  da.num_slices = cache->num_slices;
  da.cap = cache->cap;
  da.max_len = cache->max_len;
  da.H_q = H_q;
  da.H_kv = H_kv;
  da.tsplit = ts;
  da.scale_log2 = scale_log2;
  da.err = a.err;
  da.item_off = a.item_off;
  da.item_zp = a.item_zp;
  da.part = reinterpret_cast<float *>(w + lay.part);
  e = csmkv::launch_decode_table(da, cache->dtype, cache->d, G, lay.items, st);
  return e ? CSMKV_EHIP : CSMKV_OK;
}

int csmkv_clear_error(int32_t *error_word, void *stream) {
  if (error_word == nullptr || !aligned(error_word, 4)) return CSMKV_EINVAL;
  return csmkv::launch_clear(error_word, static_cast<hipStream_t>(stream)) ? CSMKV_EHIP : CSMKV_OK;
}

int csmkv_read_error(const int32_t *error_word, void *stream) {
  if (error_word == nullptr) return CSMKV_EINVAL;
  int32_t host = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&host, error_word, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess)
    return CSMKV_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return CSMKV_EHIP;
  return host == 0 ? CSMKV_OK : CSMKV_EDEVICE;
}

}  // extern "C"
