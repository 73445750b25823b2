"""Plain, slow, fp64 CPU oracle for Chunked Soft Matching (CSM) KV-cache clustering
and log-degree decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, constants or helpers with the HIP path in
``kv_cache_clustering_amd`` and imports nothing from it.

Sources (cited by page title and section; the pages are the authority):
  * "Chelsea: Efficient Long-Context LLM Inference via KV Cache Clustering"
    (xllm-io paper review) -- section 三 技术架构: 核心公式 (the clustered-attention
    approximation and the log-N attention formula), Algorithm 1 (inference pipeline),
    分块软匹配算法 steps 1-4, 定理 6.1; section 五: default settings.
  * "CentroidKV: Efficient Long-Context LLM Inference via KV Cache Clustering"
    (gist.science) -- 技术摘要 / 方法论: 推理流水线, 分块软匹配 (CSM), 聚合.

Modules:
  bf16       -- round-to-nearest-even to bfloat16, bit conversions (definition of the format).
  csm        -- one CSM round over a cache, step by step, with decision taps.
  attention  -- log-N decode attention, plain softmax attention, cache append.
  schedule   -- Algorithm 1 budget / trigger / annealing as plain integer loops.
  theorem    -- Theorem 6.1 objective and brute-force maximiser search.
  index      -- hierarchical centroid index (ball tree) over a clustered cache and attention
                over the rows it keeps (LycheeCluster page, 层次 KV 索引 / 流式懒更新).

Parity status per function is stated in each module header.  Values of merged
centroids at specific inputs are "parity unpinned" beyond the invariants listed in
``csm``: the pages print no worked example with numbers.
"""

from . import bf16, csm, attention, schedule, theorem, index  # noqa: F401
