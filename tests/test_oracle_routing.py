"""Pins of the oracle's routing (router logits, softmax gate, group-limited top-k, weights).

Each test checks the oracle against something other than itself: a worked
example, exhaustive enumeration, a library routine on a special case, or an
invariant the definition implies.
"""
import math
import os
from fractions import Fraction
from itertools import combinations

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as mo
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ----------------------------------------------------------------- brute force definition
def _best_subset(values: dict, size: int):
    """The size-subset with the largest exact sum; ties -> lexicographically smallest index list."""
    def key(c):
        return (-sum(Fraction(values[i]) for i in c), tuple(sorted(c)))
    return sorted(min(combinations(sorted(values), size), key=key))


def _route_bruteforce(scores_row, G, Gk, k):
    s = [float(v) for v in scores_row]
    n = len(s) // G
    groups = _best_subset({g: max(s[g * n:(g + 1) * n]) for g in range(G)}, Gk)
    cand = {e: s[e] for g in groups for e in range(g * n, (g + 1) * n)}
    return _best_subset(cand, k), groups


def test_worked_example():
    g = _golden("routing_worked.txt")
    G, Gk, k = int(g["G"][0]), int(g["Gk"][0]), int(g["k"][0])
    logits = np.array([[float(v) for v in g["logits"]]])
    ids, kept = mo.select_experts(mo.gate_scores(logits), G, Gk, k)
    assert ids[0].tolist() == [int(v) for v in g["ids"]]
    assert kept[0].tolist() == [int(v) for v in g["kept_groups"]]
    w = mo.renormalise(mo.gate_scores(logits), ids)[0]
    D = 1 + math.exp(-1) + math.exp(-2.5)
    np.testing.assert_allclose(w, [1 / D, math.exp(-1) / D, math.exp(-2.5) / D], rtol=1e-14)


@pytest.mark.parametrize("G,Gk,k,E", [(4, 2, 4, 16), (4, 2, 3, 8), (2, 1, 2, 8), (4, 3, 4, 12),
                                       (1, 1, 3, 8), (4, 4, 2, 8), (3, 2, 5, 12)])
@pytest.mark.parametrize("kind", ["normal", "integer_ties"])
def test_bruteforce_enumeration(G, Gk, k, E, kind):
    rng = np.random.default_rng(E * 100 + G * 10 + k)
    for _ in range(60):
        if kind == "normal":
            logits = rng.standard_normal((1, E))
        else:  # few distinct values -> many exact ties at both stages
            logits = rng.integers(0, 3, size=(1, E)).astype(np.float64)
        scores = mo.gate_scores(logits)
        ids, kept = mo.select_experts(scores, G, Gk, k)
        bf_ids, bf_groups = _route_bruteforce(scores[0], G, Gk, k)
        assert sorted(ids[0].tolist()) == bf_ids
        if G > 1:
            assert kept[0].tolist() == bf_groups


def test_ungrouped_equals_torch_topk():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((64, 256))
    scores = mo.gate_scores(logits)
    ids, _ = mo.select_experts(scores, 1, 1, 6)
    ref = torch.topk(torch.from_numpy(scores), 6, dim=1).indices.numpy()
    assert np.array_equal(ids, ref)


def test_keep_all_groups_equals_ungrouped():
    rng = np.random.default_rng(8)
    scores = mo.gate_scores(rng.standard_normal((32, 128)))
    a, _ = mo.select_experts(scores, 8, 8, 8)
    b, _ = mo.select_experts(scores, 1, 1, 8)
    assert np.array_equal(a, b)


def test_k1_weight_is_one_and_full_groups():
    rng = np.random.default_rng(9)
    scores = mo.gate_scores(rng.standard_normal((16, 16)))
    ids, _ = mo.select_experts(scores, 4, 2, 1)
    assert np.all(mo.renormalise(scores, ids) == 1.0)
    # Gk * n == k: every expert of the kept groups is chosen
    ids, kept = mo.select_experts(scores, 4, 2, 8)
    for t in range(16):
        members = sorted(e for g in kept[t] for e in range(4 * g, 4 * g + 4))
        assert sorted(ids[t].tolist()) == members


def test_weights_closed_form_softmax_of_selected_logits():
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((50, 128)) * 2.0
    scores = mo.gate_scores(logits)
    ids, _ = mo.select_experts(scores, 8, 4, 8)
    w = mo.renormalise(scores, ids)
    ref = scipy.special.softmax(np.take_along_axis(logits, ids, axis=1), axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-12, atol=0)


def test_softmax_matches_scipy():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((10, 64)) * 5
    np.testing.assert_allclose(mo.gate_scores(logits), scipy.special.softmax(logits, axis=1),
                               rtol=1e-13)


def test_router_logits_match_torch_linear():
    rng = np.random.default_rng(12)
    x, w, b = rng.standard_normal((5, 32)), rng.standard_normal((8, 32)), rng.standard_normal(8)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b))
    np.testing.assert_allclose(mo.router_logits(x, w, b), ref.numpy(), rtol=1e-13)


@pytest.mark.parametrize("name", ["tiny", "decode", "inkling"])
def test_invariants_on_workloads(name):
    shape = synth.WORKLOADS[name]
    if shape.T > 256:
        shape = shape.with_tokens(256)
    rng = np.random.default_rng(shape.seed)
    x = rng.standard_normal((shape.T, shape.H))
    wr = rng.standard_normal((shape.E, shape.H)) * 0.05
    ids, w, logits = mo.route(x, wr, None, shape.G, shape.Gk, shape.k)
    scores = mo.gate_scores(logits)
    n = shape.E // shape.G
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(w > 0)
    for t in range(shape.T):
        chosen = set(ids[t].tolist())
        assert len(chosen) == shape.k
        groups = {e // n for e in chosen}
        assert len(groups) <= shape.Gk
        gs = scores[t].reshape(shape.G, n).max(axis=1)
        kept = np.argsort(-gs, kind="stable")[:shape.Gk]
        assert groups <= set(kept.tolist())
        dropped = [g for g in range(shape.G) if g not in kept]
        if dropped:
            assert gs[kept].min() >= gs[dropped].max()
        others = [e for g in kept for e in range(g * n, (g + 1) * n) if e not in chosen]
        if others:
            assert scores[t, list(chosen)].min() >= scores[t, others].max()
        # order: score descending
        assert np.all(np.diff(scores[t, ids[t]]) <= 0)


def test_forced_ties_lower_index_wins():
    # duplicated router rows + equal bias give bit-identical logits, and equal group maxima
    H = 16
    rng = np.random.default_rng(13)
    wr = rng.standard_normal((16, H)) * 0.01
    wr[5] = wr[3]          # experts 3 and 5 tie
    wr[9] = wr[1]          # expert 9 (group 2) ties expert 1 (group 0)
    x = rng.standard_normal((1, H))
    bias = np.zeros(16)
    bias[[1, 9]] = 10.0
    bias[[3, 5]] = 9.0
    logits = mo.router_logits(x, wr, bias)
    assert logits[0, 1] == logits[0, 9] and logits[0, 3] == logits[0, 5]
    scores = mo.gate_scores(logits)
    # groups of 4: g0={0..3} max 10, g1={4..7} max 9, g2={8..11} max 10 -> keep 2: g0, g2
    ids, kept = mo.select_experts(scores, 4, 2, 2)
    assert kept[0].tolist() == [0, 2]
    assert ids[0].tolist() == [1, 9]
    ids, kept = mo.select_experts(scores, 4, 1, 2)   # g0 and g2 tie -> g0
    assert kept[0].tolist() == [0]
    assert ids[0].tolist() == [1, 3]
    ids, _ = mo.select_experts(scores, 1, 1, 3)      # ungrouped: 1, 9 tie at top; then 3 vs 5
    assert ids[0].tolist() == [1, 9, 3]


def test_margins_match_definition():
    g = _golden("routing_worked.txt")
    logits = np.array([[float(v) for v in g["logits"]]])
    gg, ge = mo.topk_margins(logits, 4, 2, 3)
    assert gg[0] == 0.0            # 2nd and 3rd group maxima tie at 2.0
    assert ge[0] == 0.5 - (-1.0)   # 3rd best candidate 0.5 vs 4th -1.0
    gg, ge = mo.topk_margins(logits, 1, 1, 3)
    assert gg[0] == np.inf and ge[0] == 2.0 - 1.5   # 3rd best 2.0 (e6) vs 4th 1.5 (e3)


def test_page_shapes():
    """The Ling-3.0-tiny and Inkling MoE shapes of the pages."""
    d = synth.WORKLOADS["decode"]
    assert (d.E, d.G, d.E // d.G, d.Gk, d.k, d.H) == (128, 8, 16, 4, 8, 1536)
    for name in ("prefill", "fp8"):
        s = synth.WORKLOADS[name]
        assert (s.E, s.G, s.Gk, s.k, s.H, s.I) == (d.E, d.G, d.Gk, d.k, d.H, d.I)
    ink = synth.WORKLOADS["inkling"]
    assert (ink.E, ink.k, ink.S, ink.G) == (256, 6, 2, 1)
