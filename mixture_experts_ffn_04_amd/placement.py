"""Expert placement for expert-parallel shares (host side, run once).

The article's section "Expert Parallelism" gives each of N devices E/N of
the experts without fixing which.  A contiguous block per device leaves
each device's routed work to chance.  Under a skewed router, a few popular
experts then land together.  `balanced_shares` spreads the experts by
their measured load: the most loaded expert goes first, each to the least
loaded share that still has room.  This is the longest-processing-time-first
rule with equal expert counts per share.  `expert_map` turns one share into
the global → local table that moe_localize_ids_mapped reads.
"""
from typing import List, Sequence


def balanced_shares(loads: Sequence[float], n: int) -> List[List[int]]:
    """Split experts 0..E-1 into n shares of E // n or E // n + 1 experts
    (the first E % n shares take one more), greedily by load.

    loads[e] is expert e's routed rows in a calibration batch, or any other
    load estimate.  Experts are visited by decreasing load (ties: lower id
    first).  Each goes to the share with the least load so far among those
    below their expert count (ties: lower share index).  Each share's
    experts are returned in increasing global id, the order in which its
    packed weights hold them."""
    E = len(loads)
    if n < 1 or E < n:
        raise ValueError("balanced_shares needs 1 <= n <= number of experts")
    cap = [E // n + (1 if i < E % n else 0) for i in range(n)]
    held: List[List[int]] = [[] for _ in range(n)]
    total = [0.0] * n
    for e in sorted(range(E), key=lambda e: (-float(loads[e]), e)):
        best = min((i for i in range(n) if len(held[i]) < cap[i]), key=lambda i: (total[i], i))
        held[best].append(e)
        total[best] += float(loads[e])
    return [sorted(h) for h in held]


def expert_map(held: Sequence[int], num_experts: int) -> List[int]:
    """The global -> local table of one share: entry e is e's position in
    `held`, -1 for the experts held elsewhere."""
    m = [-1] * num_experts
    for j, e in enumerate(held):
        if not 0 <= e < num_experts or m[e] != -1:
            raise ValueError("held experts must be distinct ids in [0, num_experts)")
        m[e] = j
    return m
