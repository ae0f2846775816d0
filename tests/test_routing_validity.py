"""The near-tie validity rule of the GPU parity tests (tests/helpers.routing_invalid),
checked on the CPU: every routing the oracle produces on logits perturbed within the
margin passes, and routings with a planted mistake (a dropped leading group, a chosen
expert well below a left-out one, a group outside the kept set, a duplicate id) fail."""
import numpy as np
import pytest

from oracle import moe_oracle as mo
from tests.helpers import NEAR_TIE, routing_invalid


def _oracle_ids(l, G, Gk, k):
    ids, _ = mo.select_experts(mo.gate_scores(l[None]), G, Gk, k)
    return ids[0]


@pytest.mark.parametrize("G,Gk,k,E", [(8, 4, 8, 128), (4, 2, 4, 16), (1, 1, 6, 256), (64, 8, 16, 256)])
def test_perturbed_oracle_routings_are_valid(G, Gk, k, E):
    rng = np.random.default_rng(G * 100 + k)
    for _ in range(200):
        l = rng.standard_normal(E)
        # plant near-ties: copy values with tiny offsets so the margin is below tol
        src = rng.choice(E, 8, replace=False)
        dst = rng.choice(E, 8, replace=False)
        l[dst] = l[src] + rng.uniform(-NEAR_TIE / 3, NEAR_TIE / 3, 8)
        ids = _oracle_ids(l, G, Gk, k)
        assert routing_invalid(ids, l, G, Gk, k) is None
        # the oracle on logits moved by less than half the margin is still valid
        lp = l + rng.uniform(-NEAR_TIE / 2.5, NEAR_TIE / 2.5, E)
        assert routing_invalid(_oracle_ids(lp, G, Gk, k), l, G, Gk, k) is None


def test_planted_mistakes_fail():
    G, Gk, k, E, n = 4, 2, 4, 16, 4
    l = np.array([9.0, 1, 2, 3,   8, 7, 6, 0,   5, 4.5, 4, 3.5,   0.5, 0.4, 0.3, 0.2])
    good = _oracle_ids(l, G, Gk, k)                     # groups 0 and 1: 0, 4, 5, 6
    assert sorted(good.tolist()) == [0, 4, 5, 6]
    assert routing_invalid(good, l, G, Gk, k) is None
    # a kept group's expert swapped for a weaker one of the same group (3 < 6 by 3)
    assert "beats" in routing_invalid(np.array([0, 4, 5, 3]), l, G, Gk, k)
    # an expert from a dropped group (group 2 scores 5 < 8)
    assert "below the kept groups" in routing_invalid(np.array([0, 4, 5, 8]), l, G, Gk, k)
    # duplicate id
    assert "distinct" in routing_invalid(np.array([0, 4, 4, 5]), l, G, Gk, k)
    # a group within the margin may replace the Gk-th: groups 1 and 2 tie at 8
    l2 = l.copy()
    l2[8] = 8.0 + NEAR_TIE / 2
    assert routing_invalid(np.array([0, 8, 9, 10]), l2, G, Gk, k) is None
    assert routing_invalid(np.array([0, 1, 2, 8]), l2, G, Gk, k) is not None
    assert routing_invalid(np.array([0, 4, 5, 6]), l2, G, Gk, k) is None
    # ... but not when group 2 is clearly ahead (8.01): dropping it is wrong
    l3 = l.copy()
    l3[8] = 8.01
    assert routing_invalid(np.array([0, 4, 5, 6]), l3, G, Gk, k) is not None
    # ungrouped: a left-out logit within tol of the k-th is fine, beyond it is not
    l4 = np.array([5.0, 4.0, 3.0, 2.0 + NEAR_TIE / 2, 2.0, 1.0])
    assert routing_invalid(np.array([0, 1, 2, 4]), l4, 1, 1, 4) is None
    l4[3] = 2.0 + 3 * NEAR_TIE
    assert routing_invalid(np.array([0, 1, 2, 4]), l4, 1, 1, 4) is not None
