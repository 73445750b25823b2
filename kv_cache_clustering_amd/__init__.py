"""MI355X-native Chunked Soft Matching (CSM) KV-cache clustering and log-N decode attention.

The compute path is libcsmkv.so (hand-written HIP kernels for gfx950 behind a C ABI,
declared in include/csmkv.h).  ``kv_cache_clustering_amd._lib`` is its thin ctypes
binding (importing it fails loudly when the library is not built); ``schedule`` is the
host-side Algorithm 1 bookkeeping (budget, trigger, r annealing), pure integer logic;
``pipeline`` drives a cache through Algorithm 1 with the library.
"""

from . import schedule  # noqa: F401
