"""Expert placement over expert-parallel shares (host logic, no GPU)."""
import itertools

import numpy as np
import pytest

from mixture_experts_ffn_04_amd.placement import balanced_shares, expert_map


def _check_partition(shares, E, n):
    flat = sorted(e for h in shares for e in h)
    assert flat == list(range(E))
    assert [len(h) for h in shares] == [E // n + (1 if i < E % n else 0) for i in range(n)]
    assert all(h == sorted(h) for h in shares)


def test_hand_case():
    """Loads 5 1 9 3 7 2 8 4 over two shares of four: experts by decreasing
    load 2, 6, 4, 0, 7, 3, 5, 1 go to the lighter share with room, giving
    {0, 2, 5, 7} (load 20) and {1, 3, 4, 6} (load 19)."""
    assert balanced_shares([5, 1, 9, 3, 7, 2, 8, 4], 2) == [[0, 2, 5, 7], [1, 3, 4, 6]]


def test_equal_loads_and_one_share():
    """Equal loads: ties go to the lower share and lower expert, so the
    experts are dealt out in turn.  One share holds everything."""
    assert balanced_shares([1.0] * 8, 4) == [[0, 4], [1, 5], [2, 6], [3, 7]]
    assert balanced_shares([3, 0, 2], 1) == [[0, 1, 2]]


def test_uneven_counts_and_errors():
    s = balanced_shares(list(range(10)), 3)
    _check_partition(s, 10, 3)
    with pytest.raises(ValueError):
        balanced_shares([1, 2], 3)
    with pytest.raises(ValueError):
        balanced_shares([1, 2], 0)


@pytest.mark.parametrize("E,n,seed", [(8, 2, 0), (8, 4, 1), (9, 3, 2), (12, 3, 3), (12, 4, 4), (10, 2, 5)])
def test_against_brute_force(E, n, seed):
    """On Zipf-like loads small enough to enumerate every placement with
    equal expert counts, the greedy placement's heaviest share is within
    a third of the optimum (and never below it)."""
    rng = np.random.default_rng(seed)
    loads = (rng.permutation(E) + 1.0) ** -1.0 * 1000 + rng.integers(0, 5, E)
    shares = balanced_shares(loads, n)
    _check_partition(shares, E, n)
    got = max(sum(loads[e] for e in h) for h in shares)
    size = E // n
    best = float("inf")

    def search(left, groups):
        nonlocal best
        if not left:
            best = min(best, max(sum(loads[e] for e in g) for g in groups))
            return
        first = left[0]
        for rest in itertools.combinations(left[1:], size - 1):
            g = (first,) + rest
            search([e for e in left if e not in g], groups + [g])

    search(list(range(E)), [])
    assert best <= got <= best * 4 / 3 + 1e-9


def test_zipf_spreads_hot_experts():
    """256 experts with Zipf(1.0) loads over 8 shares of 32.  The share that
    holds the hottest expert carries at least that expert plus the 31
    lightest, which here exceeds the mean; the greedy placement reaches
    that bound exactly, below contiguous blocks and every-8th-expert
    shares of the same loads."""
    rng = np.random.default_rng(7)
    E, n = 256, 8
    loads = 1e6 / (rng.permutation(E) + 1.0)
    shares = balanced_shares(loads, n)
    _check_partition(shares, E, n)
    srt = np.sort(loads)
    bound = max(loads.sum() / n, srt[-1] + srt[:E // n - 1].sum())
    worst = max(loads[h].sum() for h in shares)
    assert worst == pytest.approx(bound, rel=1e-12)
    blocks = max(loads[i * 32:(i + 1) * 32].sum() for i in range(n))
    strided = max(loads[i::n].sum() for i in range(n))
    assert worst < blocks and worst < strided


def test_expert_map():
    m = expert_map([5, 2, 7], 8)
    assert m == [-1, -1, 1, -1, -1, 0, -1, 2]
    with pytest.raises(ValueError):
        expert_map([1, 1], 4)
    with pytest.raises(ValueError):
        expert_map([4], 4)
