"""Oracle: the parallel-vs-sequential greedy decoding theorem, by brute force.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

ccyt168.com Fast-dLLM article, section 1.2 "Confidence-Aware Parallel Decoding": under
greedy decoding, if n tokens are decoded in parallel and each has confidence above
1 - eps with (n+1) eps <= 1, parallel decoding gives the same result as sequential
decoding.  The same section's poker-hands example shows why decoding positions
independently from their marginals can produce a combination the joint never favours.

Reading of "sequential decoding" (not defined on the page): chain-rule greedy on the
exact joint distribution, x1 = argmax p(X1), x2 = argmax p(X2 | x1), ... in a given
position order.  "Parallel decoding": every position takes the argmax of its own
marginal, which is what the threshold rule in ``decode`` does to the positions it
selects.
"""
from __future__ import annotations

import itertools

import numpy as np


def marginals(p: np.ndarray):
    """List of per-position marginal distributions of a joint p over V^n."""
    n = p.ndim
    return [p.sum(axis=tuple(a for a in range(n) if a != i)) for i in range(n)]


def parallel_greedy(p: np.ndarray):
    return tuple(int(np.argmax(mg)) for mg in marginals(p))


def sequential_greedy(p: np.ndarray, order=None):
    """Chain-rule greedy decoding of the joint p in the given position order."""
    n = p.ndim
    order = list(range(n)) if order is None else list(order)
    fixed: dict[int, int] = {}
    for pos in order:
        # conditional of X_pos given the positions fixed so far (unnormalised)
        idx = tuple(fixed.get(a, slice(None)) for a in range(n))
        sub = p[idx]                                   # axes: remaining free positions
        free = [a for a in range(n) if a not in fixed]
        ax = free.index(pos)
        cond = sub.sum(axis=tuple(i for i in range(len(free)) if i != ax))
        fixed[pos] = int(np.argmax(cond))
    return tuple(fixed[a] for a in range(n))


def joint_mode(p: np.ndarray):
    return tuple(int(i) for i in np.unravel_index(int(np.argmax(p)), p.shape))


def condition_holds(p: np.ndarray) -> tuple[bool, float]:
    """(n+1) eps <= 1 with eps the smallest value such that every marginal max > 1 - eps.

    Since the condition needs a strict inequality, eps is taken just above
    1 - min_i max_x p_i(x).
    """
    n = p.ndim
    cmin = min(float(mg.max()) for mg in marginals(p))
    eps = np.nextafter(1.0 - cmin, 2.0)
    return (n + 1) * eps <= 1.0, float(eps)


def all_orders(n: int):
    return list(itertools.permutations(range(n)))
