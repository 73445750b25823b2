"""Seeded synthetic K/V caches, queries and appended tokens.

This module serves both the GPU path's tests and benchmark and the oracle's tests, and
holds none of the clustering or attention arithmetic: only random draws, the AR(1)
key process that stands in for real key states, and the workload shapes.

Stand-in statement: the pages measure on Llama-family models with public long-context
suites.  No model weights or suite items are used here; the AR(1) keys reproduce the
two observations the method rests on (keys are locally cosine-similar, and similarity
decays convexly with token distance: CentroidKV page, 方法论 / 观察结果; Chelsea review,
section 二 关键观察 and Figure 3), and the shapes follow the models' KV layout.
"""

from .configs import WORKLOADS, Workload, workload  # noqa: F401
from .gen import (  # noqa: F401
    seed_of,
    ar1_numpy,
    make_cache,
    make_queries,
    outlier_mask,
    slice_params,
)
