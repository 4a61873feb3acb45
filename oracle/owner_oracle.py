"""CPU oracle for owner assignment.  TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/`` may import this module.  The product's assignment (``muon_owner_assign`` in
the HIP library's host code) shares no code with it.

Source: "Riepilogo Tecnico: DMuon" (Italian summary of DMuon), §2.3.  Each matrix gets one
owner rank.  The assignment minimises the predicted makespan, the largest total cost of any
one owner, and is posed as a mixed-integer program.  A greedy heuristic stands in when the
search space is too large.  The costs come from measured step times.

* ``optimal_makespan`` is the definition of the MILP's optimum: the minimum, over every
  assignment of the n matrices to the R owners, of the largest owner load.  It enumerates all
  R^n assignments, so it is for small instances only.
* ``greedy_longest_first`` is the greedy heuristic as read here.  Matrices are taken in
  decreasing cost, ties in list order.  Each goes to the owner with the smallest load so
  far, the lowest index on ties.  The pages name only "greedy"; this longest-first form is
  the classic one for minimising the makespan.

Parity status: both functions are pinned by tests/test_owner.py.  The pins are Graham's
worst cases for longest-first, with their known greedy and optimal makespans, and special
cases solvable by hand.
"""

from __future__ import annotations

import itertools


def loads_of(costs, owner, ranks: int) -> list[float]:
    """Total cost of each owner under an assignment."""
    loads = [0.0] * ranks
    for c, r in zip(costs, owner):
        loads[r] += c
    return loads


def optimal_makespan(costs, ranks: int):
    """(makespan, owner) minimising the largest owner load, by exhaustive enumeration.

    Among optimal assignments the first in lexicographic order of ``owner`` is returned.
    """
    costs = [float(c) for c in costs]
    if not costs:
        return 0.0, []
    best, best_owner = None, None
    for owner in itertools.product(range(ranks), repeat=len(costs)):
        m = max(loads_of(costs, owner, ranks))
        if best is None or m < best:
            best, best_owner = m, list(owner)
    return best, best_owner


def greedy_longest_first(costs, ranks: int):
    """(makespan, owner) of the longest-first greedy described in the module docstring."""
    costs = [float(c) for c in costs]
    order = sorted(range(len(costs)), key=lambda i: (-costs[i], i))
    loads = [0.0] * ranks
    owner = [0] * len(costs)
    for i in order:
        r = min(range(ranks), key=lambda k: (loads[k], k))
        owner[i] = r
        loads[r] += costs[i]
    return (max(loads) if costs else 0.0), owner
