"""Host-side Algorithm 1 bookkeeping: budget, trigger, r annealing, closed-form lengths.

Chelsea review, section 三, Algorithm 1: B = R * (n + Gamma); after prefill and after
every decode append, a clustering round runs while / when s >= B + g.  CentroidKV page,
渐进式调度: r_j = r_init - j * delta_r over rounds j (floored at r_min here).

All quantities are host integers: the length after a round is known in closed form, so
driving the device never needs a read-back.  For a slice of length s:
  M = s - n1 - n2;  F = M // c full chunks;  t = M % c tail rows;
  s' = s - F * floor(r*c/2) - floor(r*t/2)   (tail term 0 when t < 2; M < 2: s' = s).
"""

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


def chunk_merges(r, L):
    """Merges in a chunk of length L: floor(r*L/2) with a 1e-9 guard, in [0, ceil(L/2)]."""
    if L < 2:
        return 0
    return max(0, min((L + 1) // 2, math.floor(r * L / 2.0 + 1e-9)))


def round_output_length(s, n1, n2, c, r):
    M = s - n1 - n2
    if M < 2:
        return s
    F, t = divmod(M, c)
    return s - F * chunk_merges(r, c) - chunk_merges(r, t)


def annealed_r(j, r_init=0.5, delta=0.05, r_min=0.1):
    return max(r_init - j * delta, r_min)


@dataclass
class Algorithm1:
    """Length bookkeeping of one sequence's cache under Algorithm 1."""
    n: int
    R: Optional[float]
    Gamma: int
    g: int = 32
    n1: int = 16
    n2: int = 64
    c: int = 256
    r_init: float = 0.5
    delta: float = 0.05
    r_min: float = 0.1
    s: int = field(init=False)
    j: int = field(init=False, default=0)
    rounds: List[Tuple[int, float, int, int]] = field(init=False, default_factory=list)

    def __post_init__(self):
        self.s = self.n

    @property
    def budget(self):
        return None if self.R is None else self.R * (self.n + self.Gamma)

    def over_budget(self):
        return self.budget is not None and self.s >= self.budget + self.g

    def next_round(self, step=0):
        """r of the round to run now (and advance the bookkeeping), or None."""
        if not self.over_budget():
            return None
        return self._round(step)

    def force_round(self, step=0):
        return self._round(step)

    def _round(self, step):
        r = annealed_r(self.j, self.r_init, self.delta, self.r_min)
        s2 = round_output_length(self.s, self.n1, self.n2, self.c, r)
        self.rounds.append((step, r, self.s, s2))
        self.s = s2
        self.j += 1
        return r

    def prefill_rounds(self):
        """Rounds run before decoding: repeated until the cache is below B + g."""
        rs = []
        while True:
            r = self.next_round(0)
            if r is None:
                return rs
            rs.append(r)

    def append(self):
        self.s += 1
