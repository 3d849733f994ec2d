"""ZigZagKV budgets: MBA per head, LMBA per layer, proportional allocation with
a per-layer floor.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources: ZigZagKV blog page (qidao123 thread 109074):

* section on ZigZagKV's new observations: MBA is the minimum number of KV
  entries needed to keep 90% of the total attention score of a head; LMBA is
  the mean MBA over a layer's heads; a higher LMBA needs a larger budget;
* section on ZigZagKV's space allocation: each layer receives a share of the
  model's total budget in proportion to its LMBA ratio, and a minimum size is
  reserved for every layer so that no layer is starved; SnapKV gives each
  layer the same B (the equal-LMBA case).

The formulas themselves were lost from the page; the readings used here:

* the attention-score vector of a head is its window-averaged importance
  (the SnapKV score row of that head), MBA = min{m : sum of the m largest
  entries >= mass * sum of all entries}, mass = 0.9;
* B_l = F + share_l of R = B_total - L*F, share_l proportional to
  LMBA_l (= M_l / Hkv with M_l = sum over the layer's heads of MBA, the
  1/Hkv cancels), with integer largest-remainder rounding, remainder ties to
  the lower layer; all arithmetic in exact integers;
* a layer whose budget exceeds the per-head capacity is clamped to it and the
  excess is re-shared over the other layers by the same rule (water-filling);
* B_l counts tokens per KV head of layer l, recent window included.
"""

import math

import numpy as np


def mba(scores, mass=0.9):
    """Minimum m such that the m largest entries of ``scores`` hold at least
    ``mass`` of their total.  Sums are exactly rounded (math.fsum)."""
    v = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    total = math.fsum(v)
    target = mass * total

    def holds(m):
        return math.fsum(v[:m]) >= target

    # holds(m) is monotone in m because every entry is >= 0: binary search
    # for the smallest m that holds.
    lo, hi = 0, v.size
    while lo < hi:
        mid = (lo + hi) // 2
        if holds(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _largest_remainder(R, weights):
    """Split R integer units in proportion to integer ``weights``:
    q_l = floor(R*w_l/W) plus one unit each for the R - sum(q) layers with the
    largest R*w_l mod W (ties to the lower index)."""
    W = sum(weights)
    if W == 0:
        weights = [1] * len(weights)
        W = len(weights)
    q = [(R * wl) // W for wl in weights]
    rem = [(R * wl) % W for wl in weights]
    left = R - sum(q)
    order = sorted(range(len(weights)), key=lambda l: (-rem[l], l))
    for l in order[:left]:
        q[l] += 1
    return q


def allocate(layer_sums, total_budget, floor, capacity):
    """Per-layer budgets B_l (tokens per KV head, recent included).

    layer_sums: M_l per layer (ints); total_budget: B_total; floor: F;
    capacity: max tokens a head of any layer can keep.
    """
    L = len(layer_sums)
    if floor > capacity or total_budget < L * floor or total_budget > L * capacity:
        raise ValueError("infeasible budget")
    B = [None] * L
    free = list(range(L))
    while True:
        R = total_budget - L * floor - sum(capacity - floor for l in range(L) if B[l] is not None)
        q = _largest_remainder(R, [int(layer_sums[l]) for l in free])
        over = [l for l, ql in zip(free, q) if floor + ql > capacity]
        if not over:
            for l, ql in zip(free, q):
                B[l] = floor + ql
            return B
        for l in over:
            B[l] = capacity
        free = [l for l in free if l not in over]


def zigzag_budgets(importance_model, *, total_budget, floor, capacity, mass=0.9):
    """importance_model: [L, Hkv, n] (layer, KV head, prefix token).

    MBA per (layer, head); M_l = sum over the layer's heads of MBA (LMBA_l =
    M_l / Hkv; the 1/Hkv cancels in the proportional share, so the exact
    integer sum is what the allocation weighs).  Returns (mba [L][Hkv] ints,
    budgets [L] ints)."""
    imp = np.asarray(importance_model, dtype=np.float64)
    if imp.ndim != 3:
        raise ValueError("importance must be [L, Hkv, n]")
    mbas = [[mba(imp[l, g], mass) for g in range(imp.shape[1])] for l in range(imp.shape[0])]
    sums = [sum(mbas[l]) for l in range(imp.shape[0])]
    return mbas, allocate(sums, total_budget, floor, capacity)
