"""Pins of the owner-assignment oracle against values fixed by the mathematics.

The worst cases of the longest-first greedy (Graham, "Bounds on multiprocessing timing
anomalies", 1969) have known greedy and optimal makespans.  There are 2R + 1 jobs: two each
of lengths 2R-1, 2R-2, ..., R+1, and three of length R.  The greedy makespan is 4R - 1; the
optimum is 3R.  The remaining pins are special cases solvable by hand.
"""

from __future__ import annotations

import itertools
import random

import pytest

from oracle.owner_oracle import greedy_longest_first, loads_of, optimal_makespan


def graham_instance(R: int) -> list[int]:
    jobs = []
    for length in range(2 * R - 1, R, -1):
        jobs += [length, length]
    return jobs + [R, R, R]


@pytest.mark.parametrize("R", [2, 3])
def test_graham_worst_case(R):
    jobs = graham_instance(R)
    assert len(jobs) == 2 * R + 1
    g, _ = greedy_longest_first(jobs, R)
    assert g == 4 * R - 1
    opt, owner = optimal_makespan(jobs, R)
    assert opt == 3 * R
    assert max(loads_of(jobs, owner, R)) == opt


def test_hand_cases():
    # Two owners, {5, 4, 3, 3, 3}: 5 + 4 = 3 + 3 + 3 = 9 is a perfect split.
    assert optimal_makespan([5, 4, 3, 3, 3], 2)[0] == 9
    # One owner: the total.  At least as many owners as matrices: the largest matrix.
    assert optimal_makespan([2, 7, 1], 1)[0] == 10
    assert optimal_makespan([2, 7, 1], 3)[0] == 7
    assert optimal_makespan([2, 7, 1], 5)[0] == 7
    # Equal costs over R owners: ceil(n / R) of them on the busiest owner.
    assert optimal_makespan([1] * 7, 3)[0] == 3
    assert greedy_longest_first([1] * 7, 3)[0] == 3
    assert optimal_makespan([], 4) == (0.0, [])
    assert greedy_longest_first([0, 0, 0], 2)[0] == 0


def test_greedy_tie_rules():
    # Equal costs go round robin to owners 0, 1, 2, ... in list order.
    _, owner = greedy_longest_first([4, 4, 4, 4], 3)
    assert owner == [0, 1, 2, 0]
    # Larger costs first: the 9 is placed before the earlier 1s.
    _, owner = greedy_longest_first([1, 1, 9], 2)
    assert owner[2] == 0 and owner[:2] == [1, 1]


def test_optimum_brackets_and_greedy_bound():
    """Lower bounds max(cost) and total / R; Graham's bound greedy <= (4/3 - 1/(3R)) opt."""
    rng = random.Random(11)
    for _ in range(150):
        R = rng.choice([2, 3])
        n = rng.randint(1, 7)
        costs = [rng.randint(0, 20) for _ in range(n)]
        opt, _ = optimal_makespan(costs, R)
        assert opt >= max(costs) and opt * R >= sum(costs)
        g, owner = greedy_longest_first(costs, R)
        assert g == max(loads_of(costs, owner, R))
        assert g * 3 * R <= (4 * R - 1) * opt + 1e-9


def test_enumeration_is_exhaustive_on_a_tiny_case():
    # Every assignment of 3 matrices to 2 owners, checked independently.
    costs = [3, 2, 2]
    best = min(max(loads_of(costs, o, 2)) for o in itertools.product(range(2), repeat=3))
    assert optimal_makespan(costs, 2)[0] == best == 4
