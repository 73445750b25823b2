"""Algorithm 1 lengths, budget, trigger and r annealing as plain integer loops.

TEST INFRASTRUCTURE ONLY.  Written from:
  * Chelsea review, section 三, Algorithm 1: inputs R, r, Gamma, n1, n2, g, c; budget
    B = R*(n + Gamma); after prefill, cluster if s >= B + g; decode loop i = 1 .. Gamma-1
    appends one token (s = s + 1), attends, then clusters if s >= B + g.
  * CentroidKV page, 方法论 / 渐进式调度: r is annealed linearly over clustering rounds,
    r = r_init - j * delta_r; the 局限 paragraph: a step removes at most half.

Readings: B is real-valued and compared as a real; the prefill test is applied
repeatedly until the cache is below B + g (the workloads say "compress to the budget");
j counts rounds from 0 for the sequence, prefill rounds included; r is floored at r_min.

The length after one round is computed here by walking the chunks and summing each
chunk's merge count (csm.merge_count); the product's host driver uses a closed form.
Pins: tests/golden/schedule_trajectories.json (lengths derived by hand from the same
algorithm and readings) and agreement with csm_round_slice's output length.
"""

from .csm import chunk_bounds, merge_count


def round_length(s, n1, n2, c, r):
    """Cache length after one CSM round: s minus the merges of every chunk."""
    removed = 0
    for (a, b) in chunk_bounds(s, n1, n2, c):
        removed += merge_count(r, b - a)
    return s - removed


def annealed_r(j, r_init=0.5, delta=0.05, r_min=0.1):
    return max(r_init - j * delta, r_min)


def run_algorithm1(n, R, Gamma, g, n1=16, n2=64, c=256, r_init=0.5, delta=0.05,
                   r_min=0.1, prefill_repeat=True):
    """Simulate the lengths of Algorithm 1.

    Returns a dict with the budget, the list of lengths after each prefill round, the
    decode trigger events (step, length before, length after, r) and the final length
    after the Gamma-1 decode steps.
    """
    B = R * (n + Gamma)
    s = n
    j = 0
    prefill = [s]
    while s >= B + g:
        s = round_length(s, n1, n2, c, annealed_r(j, r_init, delta, r_min))
        j += 1
        prefill.append(s)
        if not prefill_repeat:
            break
    triggers = []
    for i in range(1, Gamma):
        s += 1
        if s >= B + g:
            r = annealed_r(j, r_init, delta, r_min)
            s2 = round_length(s, n1, n2, c, r)
            triggers.append((i, s, s2, r))
            s = s2
            j += 1
    return {"budget": B, "prefill": prefill, "triggers": triggers, "final": s,
            "rounds": j}
