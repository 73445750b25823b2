"""The five synthetic workloads (shapes, data recipe, schedule parameters).

Slice order everywhere: slice = group * H_kv + kv_head, group = batch_index * layers + layer.
"""

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    batch: int
    layers: int
    H_kv: int
    H_q: int
    d: int
    dtype: str                      # storage / compute input type: "bf16", "f16" or "f32"
    ctx: int                        # prefill length n
    steps: int                      # Gamma: maximum decode length
    cap_extra: int                  # capacity beyond ctx reserved for appends
    R: Optional[float]              # cache budget ratio (None: one compress call, no budget)
    g: int = 32
    n1: int = 16
    n2: int = 64
    c: int = 256
    r_init: float = 0.5
    delta: float = 0.05
    r_min: float = 0.1
    rho: Tuple[float, float] = (0.95, 0.95)   # AR(1) coefficient range (uniform per head)
    sigma: Optional[float] = None   # innovation scale; None -> sqrt(1 - rho^2)
    mean_std: float = 0.0           # per-head mean offset of the keys (vector, iid entries)
    outlier_frac: float = 0.0
    append: bool = True             # decode steps append a token before attending

    @property
    def groups(self):
        return self.batch * self.layers

    @property
    def slices(self):
        return self.groups * self.H_kv

    @property
    def cap(self):
        return self.ctx + self.cap_extra

    @property
    def G(self):
        return self.H_q // self.H_kv


WORKLOADS = {
    1: Workload(1, "single-head-2k-fp32", batch=1, layers=1, H_kv=1, H_q=1, d=128,
                dtype="f32", ctx=2048, steps=1, cap_extra=0, R=None, sigma=0.31,
                append=False),
    2: Workload(2, "llama3-8b-16k-bf16", batch=1, layers=32, H_kv=8, H_q=32, d=128,
                dtype="bf16", ctx=16384, steps=64, cap_extra=64, R=None, mean_std=0.5),
    3: Workload(3, "llama3-8b-32k-b4-budget20-decode1000", batch=4, layers=32, H_kv=8,
                H_q=32, d=128, dtype="bf16", ctx=32768, steps=1000, cap_extra=1000, R=0.2),
    4: Workload(4, "llama3-8b-64k-budget20-outlier4", batch=1, layers=32, H_kv=8, H_q=32,
                d=128, dtype="bf16", ctx=65536, steps=256, cap_extra=256, R=0.2,
                rho=(0.8, 0.99), outlier_frac=0.04),
    5: Workload(5, "llama2-7b-32k-mha-b8-budget25", batch=8, layers=32, H_kv=32, H_q=32,
                d=128, dtype="bf16", ctx=32768, steps=128, cap_extra=128, R=0.25),
}


def workload(cid, **overrides):
    """A workload by id, optionally with fields replaced (e.g. a smaller ctx for tests)."""
    import dataclasses
    return dataclasses.replace(WORKLOADS[cid], **overrides)
