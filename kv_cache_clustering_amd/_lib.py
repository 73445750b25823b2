"""ctypes binding of libcsmkv.so: argument marshalling from torch tensors to the C ABI.

Every computation runs in the library's HIP kernels; this module only checks tensor
shapes and dtypes, builds the cache descriptor, passes device pointers and the current
HIP stream, and allocates workspaces with torch when the caller does not pass one.
Importing it fails loudly when the library has not been built.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsmkv.so")

OK, EINVAL, EDTYPE, EUNSUPPORTED, EWORKSPACE, EHIP, EDEVICE = 0, -1, -2, -3, -4, -5, -6
BF16, F32, F16 = 0, 1, 2


class CsmkvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_slices", ctypes.c_int64), ("cap", ctypes.c_int64), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_len", ctypes.c_int32)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcsmkv.so is not built ({LIB_PATH}); run "
                      "`python -c 'import __graft_entry__ as g; g.build()'` first")
_lib = ctypes.CDLL(LIB_PATH)

_p, _i32, _i64, _sz, _d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
_desc = ctypes.POINTER(CacheDesc)
_SIGS = {
    "csmkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csmkv_version": (ctypes.c_int, []),
    "csm_compress_workspace_bytes": (_sz, [_desc, _i32, _i32, _i32]),
    "csm_compress_units": (_i64, [_desc, _i32, _i32, _i32]),
    "csm_compress": (ctypes.c_int, [_p, _p, _p, _p, _desc, _i32, _i32, _i32, _d, _p, _p, _sz, _p]),
    "csm_compress_into": (ctypes.c_int, [_p, _p, _p, _p, _desc, _p, _p, _p, _p, _desc, _i32, _i32,
                                         _i32, _d, _p, _p, _sz, _p]),
    "csm_compress_debug": (ctypes.c_int, [_p, _p, _p, _p, _desc, _i32, _i32, _i32, _d, _p, _p, _sz,
                                          _p, _p, _p, _p]),
    "csm_compress_triggered": (ctypes.c_int, [_p, _p, _p, _p, _desc, _i32, _i32, _i32, _p, _p, _d,
                                              _d, _d, _p, _p, _sz, _p]),
    "decode_attn_logn_workspace_bytes": (_sz, [_desc, _i32, _i32]),
    "decode_attn_logn": (ctypes.c_int, [_p, _p, _p, _p, _p, _desc, _i32, _i32, _p, _p, _sz, _p]),
    "decode_attn_logn_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _desc, _i32, _i32, _p, _p, _p]),
    "kv_append_decode_attn_logn": (ctypes.c_int, [_p, _p, _p, _p, _p, _desc, _i32, _i32, _p, _p,
                                                  _p, _p, _sz, _p]),
    "kv_append": (ctypes.c_int, [_p, _p, _p, _p, _desc, _p, _p, _p, _p]),
    "csm_host_isa": (ctypes.c_int, []),
    "csm_compress_host": (ctypes.c_int, [_p, _p, _p, _p, _desc, _i32, _i32, _i32, _d, _p, _i32, _p,
                                         _p, _p]),
    "csm_upload_rows": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _desc, _i32, _p, _p]),
    "csm_index_bytes": (_sz, [_desc, _i32]),
    "csm_index_build": (ctypes.c_int, [_p, _p, _p, _desc, _i32, _p, _sz, _p, _p]),
    "csm_index_append": (ctypes.c_int, [_p, _p, _p, _desc, _i32, _p, _sz, _p, _p]),
    "decode_attn_logn_pruned_workspace_bytes": (_sz, [_desc, _i32, _i32, _i32]),
    "decode_attn_logn_pruned": (ctypes.c_int, [_p, _p, _p, _p, _p, _desc, _i32, _i32, _i32, _i32,
                                               _i32, _p, _sz, _d, _p, _p, _p, _sz, _p]),
    "csmkv_read_error": (ctypes.c_int, [_p, _p]),
    "csmkv_clear_error": (ctypes.c_int, [_p, _p]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def status_string(status):
    return _lib.csmkv_status_string(int(status)).decode()


def version():
    return _lib.csmkv_version()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"cache dtype must be bfloat16, float16 or float32, got {t.dtype}")


def cache_desc(K, max_len=None):
    """Descriptor of a [num_slices, cap, d] cache tensor; max_len defaults to cap."""
    if K.dim() != 3:
        raise ValueError("K must be [num_slices, cap, d]")
    S, cap, d = K.shape
    return CacheDesc(S, cap, d, _dtype_code(K), cap if max_len is None else int(max_len))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_cache(K, V, N, lens):
    if not V.is_cuda:
        raise ValueError("cache tensors must be on the GPU")
    if K.shape != V.shape or K.dtype != V.dtype:
        raise ValueError("K and V must have the same shape and dtype")
    if not V.is_contiguous():
        raise ValueError("cache tensors must be contiguous")
    _check_keys(K, N, lens)


def _check_keys(K, N, lens):
    if not (K.is_cuda and N.is_cuda and lens.is_cuda):
        raise ValueError("cache tensors must be on the GPU")
    if K.dim() != 3:
        raise ValueError("K must be [num_slices, cap, d]")
    if N.shape != K.shape[:2] or N.dtype != torch.int32:
        raise ValueError("N must be int32 [num_slices, cap]")
    if lens.shape != K.shape[:1] or lens.dtype != torch.int32:
        raise ValueError("lens must be int32 [num_slices]")
    for t in (K, N, lens):
        if not t.is_contiguous():
            raise ValueError("cache tensors must be contiguous")


def _check_mask(mask, S):
    if mask is None:
        return
    if mask.dtype != torch.uint8 or mask.shape != (S,) or not mask.is_cuda or not mask.is_contiguous():
        raise ValueError("outlier_mask must be a contiguous uint8 GPU tensor [num_slices]")


def new_workspace(nbytes, device):
    """A workspace of at least nbytes with its (sticky) error word at 0."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _workspace(nbytes, device, ws):
    if ws is None:
        return new_workspace(nbytes, device)
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous() or ws.numel() < nbytes:
        raise ValueError(f"workspace must be a contiguous uint8 GPU tensor of at least {nbytes} bytes")
    return ws


def _check_word(error_word, allow_none=False):
    if error_word is None and allow_none:
        return
    if error_word is None or error_word.dtype != torch.int32 or not error_word.is_cuda:
        raise ValueError("error_word must be an int32 GPU tensor")


def _raise(rc, what):
    if rc != OK:
        raise CsmkvError(rc, what)


def csm_workspace_bytes(K, n1, n2, c, max_len=None):
    return _lib.csm_compress_workspace_bytes(ctypes.byref(cache_desc(K, max_len)), n1, n2, c)


def csm_units(K, n1, n2, c, max_len=None):
    return _lib.csm_compress_units(ctypes.byref(cache_desc(K, max_len)), n1, n2, c)


def csm_compress(K, V, N, lens, n1=16, n2=64, c=256, r=0.5, outlier_mask=None, max_len=None,
                 workspace=None):
    """One CSM round over every slice, in place.  Returns the workspace used."""
    _check_cache(K, V, N, lens)
    _check_mask(outlier_mask, K.shape[0])
    desc = cache_desc(K, max_len)
    ws = _workspace(_lib.csm_compress_workspace_bytes(ctypes.byref(desc), n1, n2, c), K.device,
                    workspace)
    rc = _lib.csm_compress(_ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), n1, n2, c,
                           float(r), _ptr(outlier_mask), _ptr(ws), ws.numel(), _stream(K.device))
    _raise(rc, "csm_compress")
    return ws


def csm_compress_triggered(K, V, N, lens, threshold, round_index, n1=16, n2=64, c=256,
                           r_init=0.5, r_delta=0.05, r_min=0.1, outlier_mask=None, max_len=None,
                           workspace=None):
    """csm_compress in place where each slice runs only when lens >= threshold, with
    r = max(r_init - j * r_delta, r_min) from its round counter j (incremented on the device).
    threshold, round_index: int32 GPU tensors [num_slices].  Returns the workspace used."""
    _check_cache(K, V, N, lens)
    _check_mask(outlier_mask, K.shape[0])
    for t, name in ((threshold, "threshold"), (round_index, "round_index")):
        if (t is None or t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()
                or t.shape != (K.shape[0],)):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor [{K.shape[0]}]")
    desc = cache_desc(K, max_len)
    ws = _workspace(_lib.csm_compress_workspace_bytes(ctypes.byref(desc), n1, n2, c), K.device,
                    workspace)
    rc = _lib.csm_compress_triggered(_ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), n1,
                                     n2, c, _ptr(threshold), _ptr(round_index), float(r_init),
                                     float(r_delta), float(r_min), _ptr(outlier_mask), _ptr(ws),
                                     ws.numel(), _stream(K.device))
    _raise(rc, "csm_compress_triggered")
    return ws


def csm_compress_into(K_in, V_in, N_in, lens_in, K_out, V_out, N_out, lens_out, n1=16, n2=64,
                      c=256, r=0.5, outlier_mask=None, max_len=None, workspace=None):
    """One CSM round reading the first cache and writing the second."""
    _check_cache(K_in, V_in, N_in, lens_in)
    _check_cache(K_out, V_out, N_out, lens_out)
    _check_mask(outlier_mask, K_in.shape[0])
    src = cache_desc(K_in, max_len)
    dst = cache_desc(K_out, min(K_out.shape[1], src.max_len))
    ws = _workspace(_lib.csm_compress_workspace_bytes(ctypes.byref(src), n1, n2, c), K_in.device,
                    workspace)
    rc = _lib.csm_compress_into(_ptr(K_in), _ptr(V_in), _ptr(N_in), _ptr(lens_in),
                                ctypes.byref(src), _ptr(K_out), _ptr(V_out), _ptr(N_out),
                                _ptr(lens_out), ctypes.byref(dst), n1, n2, c, float(r),
                                _ptr(outlier_mask), _ptr(ws), ws.numel(), _stream(K_in.device))
    _raise(rc, "csm_compress_into")
    return ws


def csm_compress_debug(K, V, N, lens, n1=16, n2=64, c=256, r=0.5, outlier_mask=None,
                       max_len=None, workspace=None):
    """csm_compress in place, returning the decision taps (best_b, selected, src_pos)."""
    _check_cache(K, V, N, lens)
    _check_mask(outlier_mask, K.shape[0])
    desc = cache_desc(K, max_len)
    units = _lib.csm_compress_units(ctypes.byref(desc), n1, n2, c)
    S, cap = K.shape[0], K.shape[1]
    W = 128 if c <= 256 else 256  # A rows per chunk in the tap layout
    best_b = torch.full((S, max(units, 1), W), -1, dtype=torch.int32, device=K.device)
    selected = torch.zeros((S, max(units, 1), W), dtype=torch.uint8, device=K.device)
    src_pos = torch.full((S, cap), -1, dtype=torch.int32, device=K.device)
    ws = _workspace(_lib.csm_compress_workspace_bytes(ctypes.byref(desc), n1, n2, c), K.device,
                    workspace)
    rc = _lib.csm_compress_debug(_ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), n1,
                                 n2, c, float(r), _ptr(outlier_mask), _ptr(ws), ws.numel(),
                                 _stream(K.device), _ptr(best_b), _ptr(selected), _ptr(src_pos))
    _raise(rc, "csm_compress_debug")
    return best_b, selected, src_pos, ws


def decode_workspace_bytes(K, H_q, H_kv, max_len=None):
    return _lib.decode_attn_logn_workspace_bytes(ctypes.byref(cache_desc(K, max_len)), H_q, H_kv)


def decode_attn_logn(q, K, V, N, lens, H_q, H_kv, out=None, max_len=None, workspace=None):
    """O = softmax(q K^T / sqrt(d) + log N) V for every query head; O is fp32 [groups, H_q, d]."""
    _check_cache(K, V, N, lens)
    S, cap, d = K.shape
    groups = S // H_kv if H_kv > 0 else 0
    if q.shape != (groups, H_q, d) or q.dtype != K.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {K.dtype} GPU tensor [{groups}, {H_q}, {d}]")
    if out is None:
        out = torch.empty((groups, H_q, d), dtype=torch.float32, device=K.device)
    elif (out.shape != (groups, H_q, d) or out.dtype != torch.float32 or not out.is_contiguous()
          or not out.is_cuda):
        raise ValueError("out must be a contiguous fp32 GPU tensor [groups, H_q, d]")
    desc = cache_desc(K, max_len)
    ws = _workspace(_lib.decode_attn_logn_workspace_bytes(ctypes.byref(desc), H_q, H_kv),
                    K.device, workspace)
    rc = _lib.decode_attn_logn(_ptr(q), _ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc),
                               H_q, H_kv, _ptr(out), _ptr(ws), ws.numel(), _stream(K.device))
    _raise(rc, "decode_attn_logn")
    return out


def kv_append_decode_attn_logn(q, K, V, N, lens, H_q, H_kv, k_new, v_new, out=None, max_len=None,
                               workspace=None):
    """One decode step in one call: every slice appends (k_new, v_new) with degree 1, then
    attends; O is fp32 [groups, H_q, d].  max_len bounds the lengths after the append."""
    _check_cache(K, V, N, lens)
    S, cap, d = K.shape
    groups = S // H_kv if H_kv > 0 else 0
    if q.shape != (groups, H_q, d) or q.dtype != K.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {K.dtype} GPU tensor [{groups}, {H_q}, {d}]")
    for t in (k_new, v_new):
        if t.shape != (S, d) or t.dtype != K.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"k_new / v_new must be contiguous {K.dtype} GPU tensors [{S}, {d}]")
    if out is None:
        out = torch.empty((groups, H_q, d), dtype=torch.float32, device=K.device)
    elif (out.shape != (groups, H_q, d) or out.dtype != torch.float32 or not out.is_contiguous()
          or not out.is_cuda):
        raise ValueError("out must be a contiguous fp32 GPU tensor [groups, H_q, d]")
    desc = cache_desc(K, max_len)
    ws = _workspace(_lib.decode_attn_logn_workspace_bytes(ctypes.byref(desc), H_q, H_kv),
                    K.device, workspace)
    rc = _lib.kv_append_decode_attn_logn(_ptr(q), _ptr(K), _ptr(V), _ptr(N), _ptr(lens),
                                         ctypes.byref(desc), H_q, H_kv, _ptr(k_new), _ptr(v_new),
                                         _ptr(out), _ptr(ws), ws.numel(), _stream(K.device))
    _raise(rc, "kv_append_decode_attn_logn")
    return out, ws


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_attn_logn_noalloc(q, K, V, N, lens, H_q, H_kv, out, error_word, max_len=None):
    """decode_attn_logn without a workspace and without allocating anything: the library's fixed
    per-GPU scratch array holds the partials.  out (fp32 [groups, H_q, d]) and error_word (int32
    GPU tensor, sticky) are the caller's.  Calls that overlap on one GPU must not be made."""
    _check_cache(K, V, N, lens)
    S, cap, d = K.shape
    groups = S // H_kv if H_kv > 0 else 0
    if q.shape != (groups, H_q, d) or q.dtype != K.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {K.dtype} GPU tensor [{groups}, {H_q}, {d}]")
    if (out.shape != (groups, H_q, d) or out.dtype != torch.float32 or not out.is_contiguous()
            or not out.is_cuda):
        raise ValueError("out must be a contiguous fp32 GPU tensor [groups, H_q, d]")
    _check_word(error_word)
    desc = cache_desc(K, max_len)
    rc = _lib.decode_attn_logn_noalloc(_ptr(q), _ptr(K), _ptr(V), _ptr(N), _ptr(lens),
                                       ctypes.byref(desc), H_q, H_kv, _ptr(out), _ptr(error_word),
                                       _stream(K.device))
    _raise(rc, "decode_attn_logn_noalloc")
    return out


def kv_append(K, V, N, lens, k_new, v_new, error_word=None):
    """Append one token per slice: K[s]=k, V[s]=v, N[s]=1, s+=1."""
    _check_cache(K, V, N, lens)
    _check_word(error_word, allow_none=True)
    S, _, d = K.shape
    for t in (k_new, v_new):
        if t.shape != (S, d) or t.dtype != K.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"k_new / v_new must be contiguous {K.dtype} GPU tensors [{S}, {d}]")
    desc = cache_desc(K)
    rc = _lib.kv_append(_ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), _ptr(k_new),
                        _ptr(v_new), _ptr(error_word), _stream(K.device))
    _raise(rc, "kv_append")


HOST_ISA = {0: "scalar", 1: "avx2", 2: "avx512"}


def host_isa():
    """Vector unit the host round uses on this CPU: 'avx512', 'avx2' or 'scalar'."""
    return HOST_ISA[_lib.csm_host_isa()]


def _check_host(*ts):
    for t in ts:
        if t is not None and (t.is_cuda or not t.is_contiguous()):
            raise ValueError("host-round tensors must be contiguous CPU tensors")


def csm_compress_host(K, V, N, lens, n1=16, n2=64, c=256, r=0.5, outlier_mask=None, threads=0,
                      taps=False, max_len=None):
    """One CSM round in place over a cache in host memory (CPU tensors), on `threads` host
    threads (0 = all).  With taps=True returns (best_b, selected, src_pos) host tensors laid out
    as csm_compress_debug's; else None."""
    _check_host(K, V, N, lens, outlier_mask)
    if K.shape != V.shape or K.dtype != V.dtype or N.shape != K.shape[:2] or N.dtype != torch.int32:
        raise ValueError("K, V [num_slices, cap, d] of one dtype; N int32 [num_slices, cap]")
    if lens.shape != K.shape[:1] or lens.dtype != torch.int32:
        raise ValueError("lens must be int32 [num_slices]")
    if outlier_mask is not None and (outlier_mask.dtype != torch.uint8 or outlier_mask.shape != K.shape[:1]):
        raise ValueError("outlier_mask must be uint8 [num_slices]")
    desc = cache_desc(K, max_len)
    best = sel = src = None
    if taps:
        S, cap = K.shape[0], K.shape[1]
        units = _lib.csm_compress_units(ctypes.byref(desc), n1, n2, c)
        W = 128 if c <= 256 else 256
        best = torch.full((S, max(units, 1), W), -1, dtype=torch.int32)
        sel = torch.zeros((S, max(units, 1), W), dtype=torch.uint8)
        src = torch.full((S, cap), -1, dtype=torch.int32)
    rc = _lib.csm_compress_host(_ptr(K), _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), n1, n2, c,
                                float(r), _ptr(outlier_mask), int(threads), _ptr(best), _ptr(sel),
                                _ptr(src))
    _raise(rc, "csm_compress_host")
    return (best, sel, src) if taps else None


def csm_upload_rows(K_host, V_host, N_host, lens_host, K, V, N, lens, row_begin=16,
                    outlier_mask=None):
    """Enqueue the copy of the host cache's rows [row_begin, lens) (K, V, N) and lens into the
    device cache, for every slice not flagged in outlier_mask (a CPU uint8 tensor or None)."""
    _check_host(K_host, V_host, N_host, lens_host, outlier_mask)
    S = K_host.shape[0] if K_host.dim() == 3 else -1
    if (K_host.dim() != 3 or V_host.shape != K_host.shape or V_host.dtype != K_host.dtype
            or N_host.shape != K_host.shape[:2] or N_host.dtype != torch.int32
            or lens_host.shape != (S,) or lens_host.dtype != torch.int32):
        raise ValueError("host cache: K, V [num_slices, cap, d] of one dtype, N int32 "
                         "[num_slices, cap], lens int32 [num_slices]")
    if outlier_mask is not None and (outlier_mask.dtype != torch.uint8 or outlier_mask.shape != (S,)):
        raise ValueError("outlier_mask must be uint8 [num_slices]")
    _check_cache(K, V, N, lens)
    if K_host.shape != K.shape or K_host.dtype != K.dtype:
        raise ValueError("host and device caches must share their geometry")
    desc = cache_desc(K)
    rc = _lib.csm_upload_rows(_ptr(K_host), _ptr(V_host), _ptr(N_host), _ptr(lens_host), _ptr(K),
                              _ptr(V), _ptr(N), _ptr(lens), ctypes.byref(desc), int(row_begin),
                              _ptr(outlier_mask), _stream(K.device))
    _raise(rc, "csm_upload_rows")


def index_leaf_slots(cap, block_rows):
    """Leaf slots P of a slice's tree: the power of two holding cap / block_rows blocks."""
    leaves = -(-int(cap) // int(block_rows))
    P = 1
    while P < leaves:
        P *= 2
    return P


def new_index(K, block_rows=64):
    """Zeroed device memory for the hierarchical index of cache K."""
    n = _lib.csm_index_bytes(ctypes.byref(cache_desc(K)), block_rows)
    if n == 0:
        raise ValueError("unsupported index geometry")
    return torch.zeros(n, dtype=torch.uint8, device=K.device)


def _check_index_mem(index):
    if index.dtype != torch.uint8 or not index.is_cuda or not index.is_contiguous():
        raise ValueError("index must be a contiguous uint8 GPU tensor (see new_index)")


def _index_call(fn, K, N, lens, index, block_rows, error_word, max_len):
    _check_keys(K, N, lens)
    _check_word(error_word)
    _check_index_mem(index)
    desc = cache_desc(K, max_len)
    rc = fn(_ptr(K), _ptr(N), _ptr(lens), ctypes.byref(desc), int(block_rows), _ptr(index),
            index.numel(), _ptr(error_word), _stream(K.device))
    _raise(rc, fn.__name__)


def index_build(K, N, lens, index, error_word, block_rows=64, max_len=None):
    """Build every slice's ball tree over its rows [0, lens)."""
    _index_call(_lib.csm_index_build, K, N, lens, index, block_rows, error_word, max_len)


def index_append(K, N, lens, index, error_word, block_rows=64):
    """Take in the row each slice just appended (lazy update)."""
    _index_call(_lib.csm_index_append, K, N, lens, index, block_rows, error_word, None)


def decode_attn_logn_pruned(q, K, V, N, lens, H_q, H_kv, index, tau, n1=16, n2=64, block_rows=64,
                            out=None, kept=False, max_len=None, workspace=None):
    """decode_attn_logn over the rows the index keeps.  Returns (O, kept [num_slices, P] uint8 or
    None)."""
    _check_cache(K, V, N, lens)
    S, cap, d = K.shape
    groups = S // H_kv if H_kv > 0 else 0
    if q.shape != (groups, H_q, d) or q.dtype != K.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError(f"q must be a contiguous {K.dtype} GPU tensor [{groups}, {H_q}, {d}]")
    if out is None:
        out = torch.empty((groups, H_q, d), dtype=torch.float32, device=K.device)
    elif (out.shape != (groups, H_q, d) or out.dtype != torch.float32 or not out.is_contiguous()
          or not out.is_cuda):
        raise ValueError("out must be a contiguous fp32 GPU tensor [groups, H_q, d]")
    _check_index_mem(index)
    desc = cache_desc(K, max_len)
    ws = _workspace(_lib.decode_attn_logn_pruned_workspace_bytes(ctypes.byref(desc), H_q, H_kv,
                                                                 block_rows), K.device, workspace)
    tap = (torch.zeros((S, index_leaf_slots(cap, block_rows)), dtype=torch.uint8, device=K.device)
           if kept else None)
    rc = _lib.decode_attn_logn_pruned(_ptr(q), _ptr(K), _ptr(V), _ptr(N), _ptr(lens),
                                      ctypes.byref(desc), H_q, H_kv, int(n1), int(n2),
                                      int(block_rows), _ptr(index), index.numel(), float(tau),
                                      _ptr(out), _ptr(tap), _ptr(ws), ws.numel(), _stream(K.device))
    _raise(rc, "decode_attn_logn_pruned")
    return out, tap, ws


def read_error(word):
    """Synchronise and read a device error word (first int32 of a workspace, or an append word).
    The word is sticky: it stays set until clear_error."""
    return _lib.csmkv_read_error(_ptr(word), _stream(word.device))


def clear_error(word):
    """Enqueue a reset of a device error word (first int32 of a workspace, or an append word)."""
    _raise(_lib.csmkv_clear_error(_ptr(word), _stream(word.device)), "csmkv_clear_error")


# Host-only entry points for argument-validation tests (no GPU work is enqueued on errors).
raw = _lib
