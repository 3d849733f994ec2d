"""Pins for the oracle's MBA / LMBA / ZigZag allocation (CPU only).

* MBA: brute force over every subset for small n (exact rationals): the
  smallest subset holding >= 90% of the mass (the 90% comes from the ZigZagKV
  page, section on its new observations); closed forms for uniform and
  one-hot vectors.
* Allocation: hand-worked largest-remainder cases; the budgets always sum to
  the total and respect the floor (ZigZagKV page, allocation section); with
  equal LMBA the split is SnapKV's uniform one (same section's closing
  remark); a crafted capacity case exercises the water-filling.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import budget

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
MASS = GOLD["mba_mass"]["mass"]


def _brute_mba(v, mass_frac=Fraction(9, 10)):
    v = [Fraction(float(x)) for x in v]
    total = sum(v)
    for m in range(len(v) + 1):
        for sub in itertools.combinations(range(len(v)), m):
            if sum(v[i] for i in sub) >= mass_frac * total:
                return m
    raise AssertionError


@pytest.mark.parametrize("seed", range(12))
def test_mba_matches_subset_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    v = rng.exponential(size=n) ** rng.uniform(0.5, 4)
    if seed % 3 == 0:          # ties
        v = np.round(v * 3) / 3 + 0.125
    # the oracle compares against mass*total in float64; keep away from knife edges
    tot = math.fsum(v)
    sv = np.sort(v)[::-1]
    cs = np.cumsum(sv)
    if np.any(np.abs(cs - 0.9 * tot) < 1e-9 * tot):
        pytest.skip("knife-edge draw")
    assert budget.mba(v, MASS) == _brute_mba(v)


@pytest.mark.parametrize("n", [1, 7, 13, 101])
def test_mba_uniform_vector(n):
    # 0.9*n is not an integer for these n, so MBA = ceil(0.9 n)
    assert budget.mba(np.full(n, 0.25), MASS) == math.ceil(0.9 * n)


def test_mba_exact_threshold_counts_as_held():
    # top-2 of (5, 4, 1) hold exactly 9 = 0.9 * 10 (0.9*10 rounds to 9.0 in double): "keep
    # 90%" is met with equality, so MBA is 2, not 3
    assert 0.9 * 10.0 == 9.0
    assert budget.mba(np.array([1.0, 5.0, 4.0]), MASS) == 2


def test_mba_one_hot_and_zero():
    v = np.zeros(50); v[17] = 3.0
    assert budget.mba(v, MASS) == 1
    assert budget.mba(np.zeros(10), MASS) == 0


def test_mba_ninety_percent_in_few_tokens():
    # 90% of the mass on 4 tokens -> MBA is 4 (the attention-concentration picture)
    v = np.full(1000, 0.1 / 996); v[[3, 50, 700, 999]] = 0.9 / 4
    assert budget.mba(v, MASS) == 4


def test_largest_remainder_hand_cases():
    # L=3, floor 0, R=10, M=(1,1,1): q = 3 each, remainders equal -> leftover to layer 0
    assert budget.allocate([1, 1, 1], total_budget=10, floor=0, capacity=100) == [4, 3, 3]
    # M=(1,2,3), R=7: shares 7/6, 14/6, 21/6 -> q=(1,2,3), remainders (1,2,3) mod 6 -> +1 to layer 2
    assert budget.allocate([1, 2, 3], total_budget=7, floor=0, capacity=100) == [1, 2, 4]
    # with a floor of 5 on top: R = 22 - 15 = 7 -> same split plus the floor
    assert budget.allocate([1, 2, 3], total_budget=22, floor=5, capacity=100) == [6, 7, 9]


def test_water_filling_hand_case():
    # L=3, F=1, cap=5, total 12, M=(10,1,1): first pass gives (8,2,2); layer 0 clamps
    # to 5, the other 5 units above the floors split (3,2) (tie -> lower layer).
    assert budget.allocate([10, 1, 1], total_budget=12, floor=1, capacity=5) == [5, 4, 3]


@pytest.mark.parametrize("seed", range(20))
def test_allocation_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 40))
    F = int(rng.integers(0, 200))
    cap = F + int(rng.integers(1, 3000))
    total = int(rng.integers(L * F, L * cap + 1))
    M = [int(x) for x in rng.integers(0, 5000, L)]
    B = budget.allocate(M, total_budget=total, floor=F, capacity=cap)
    assert sum(B) == total
    assert all(F <= b <= cap for b in B)


def test_equal_lmba_is_uniform_snapkv():
    # SnapKV gives every layer the same B: equal LMBA must reproduce it.
    assert budget.allocate([7] * 32, total_budget=32 * 1024, floor=128, capacity=16384) == [1024] * 32


def test_allocation_tracks_lmba_order():
    B = budget.allocate([100, 400, 200, 300], total_budget=4000, floor=100, capacity=10000)
    assert B[1] > B[3] > B[2] > B[0]


def test_infeasible_budget_raises():
    with pytest.raises(ValueError):
        budget.allocate([1, 1], total_budget=5, floor=3, capacity=10)
    with pytest.raises(ValueError):
        budget.allocate([1, 1], total_budget=30, floor=3, capacity=10)


# ---- the composition the GPU budgets are compared against -----------------
def _hand_model():
    """[L=3, Hkv=2, n=7] with MBA fixed by construction (ZigZagKV page, new
    observations section: MBA is the fewest entries holding 90% of a head's
    attention): one-hot -> 1, two equal spikes -> 2 (one spike holds only 50%),
    uniform over 7 -> ceil(0.9 * 7) = 7."""
    n = 7
    one_hot = np.zeros(n); one_hot[4] = 1.0
    two_hot = np.zeros(n); two_hot[[1, 5]] = 0.5
    uniform = np.full(n, 1.0 / n)
    model = np.stack([
        np.stack([one_hot, two_hot]),     # layer 0: MBA (1, 2) -> M_0 = 3
        np.stack([uniform, one_hot]),     # layer 1: MBA (7, 1) -> M_1 = 8
        np.stack([uniform, two_hot]),     # layer 2: MBA (7, 2) -> M_2 = 9
    ])
    return model


def test_zigzag_budgets_hand_worked_exact_shares():
    # F = 2, R = 26 - 3*2 = 20, sum M = 20: shares are exactly M_l -> B = F + (3, 8, 9)
    mbas, B = budget.zigzag_budgets(_hand_model(), total_budget=26, floor=2, capacity=100, mass=MASS)
    assert mbas == [[1, 2], [7, 1], [7, 2]]
    assert B == [5, 10, 11]


def test_zigzag_budgets_hand_worked_largest_remainder():
    # F = 2, R = 19 - 6 = 13, sum M = 20: 13*M_l = 39, 104, 117 -> q = (1, 5, 5),
    # remainders (19, 4, 17) mod 20, two units left -> layers 0 and 2: q = (2, 5, 6)
    mbas, B = budget.zigzag_budgets(_hand_model(), total_budget=19, floor=2, capacity=100, mass=MASS)
    assert B == [4, 7, 8]
    # a per-layer MEAN truncated to an integer (1, 4, 4) would give (2, 9, 9) + F = (4, 11, 11)
    # at R = 20; a transposed [Hkv, L] reading would weigh the two heads, not the three layers
    _, B20 = budget.zigzag_budgets(_hand_model(), total_budget=26, floor=2, capacity=100, mass=MASS)
    assert B20 != [4, 11, 11]


def test_zigzag_budgets_layer_order_and_head_grouping():
    # permuting the layers permutes the budgets; permuting heads inside a layer changes nothing
    model = _hand_model()
    perm = [2, 0, 1]
    _, B = budget.zigzag_budgets(model, total_budget=26, floor=2, capacity=100, mass=MASS)
    _, Bp = budget.zigzag_budgets(model[perm], total_budget=26, floor=2, capacity=100, mass=MASS)
    assert Bp == [B[l] for l in perm]
    _, Bh = budget.zigzag_budgets(model[:, ::-1], total_budget=26, floor=2, capacity=100, mass=MASS)
    assert Bh == B
    # moving a uniform head from layer 2 into layer 0 moves budget with it
    swapped = model.copy()
    swapped[0, 1], swapped[2, 0] = model[2, 0], model[0, 1]   # layer 0: MBA (1, 7); layer 2: (2, 2)
    mbas, Bs = budget.zigzag_budgets(swapped, total_budget=26, floor=2, capacity=100, mass=MASS)
    assert mbas == [[1, 7], [7, 1], [2, 2]]
    assert Bs == [10, 10, 6]


def test_zigzag_budgets_rejects_wrong_rank():
    with pytest.raises(ValueError):
        budget.zigzag_budgets(np.ones((4, 5)), total_budget=8, floor=1, capacity=5)
