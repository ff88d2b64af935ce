"""Pins of the packing oracle (oracle/packing.py): hand-worked cases, closed
forms, invariants, and the objective recomputed in exact rationals from its
definition (max over ranks of |V_r - p N_r|)."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import packing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing_hand_worked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    got = packing.best_packing(case["text"], case["image"], case["ranks"], case["capacity"])
    assert (got["dev"], got["N"], got["load"]) == (case["dev"], case["N"], case["load"])


def _rational_dev(text, image, ranks, asg):
    N = sum(text) + sum(image)
    p = Fraction(sum(image), N)
    worst = Fraction(0)
    for r in range(ranks):
        Nr = sum(text[i] + image[i] for i in range(len(text)) if asg[i] == r)
        Vr = sum(image[i] for i in range(len(text)) if asg[i] == r)
        worst = max(worst, abs(Vr - p * Nr))
    return worst


def _tiny(seed):
    g = np.random.default_rng(seed)
    S = int(g.integers(1, 8))
    R = int(g.integers(1, 4))
    text = [int(v) for v in g.integers(0, 30, S)]
    image = [int(v) if g.random() < 0.7 else 0 for v in g.integers(0, 30, S)]
    if sum(text) + sum(image) == 0:
        text[0] = 1
    cap = int(max(t + v for t, v in zip(text, image)) + g.integers(0, 60))
    return text, image, R, cap


@pytest.mark.parametrize("seed", range(12))
def test_objective_equals_its_rational_definition(seed):
    text, image, R, cap = _tiny(seed)
    got = packing.best_packing(text, image, R, cap)
    if got is None:
        return
    N = got["N"]
    for asg in got["optimal"]:
        assert _rational_dev(text, image, R, asg) * N == got["dev"]
    # no feasible assignment does better, by the rational definition
    best = min(_rational_dev(text, image, R, a)
               for a in itertools.product(range(R), repeat=len(text))
               if all(sum(text[i] + image[i] for i in range(len(text)) if a[i] == r) <= cap
                      for r in range(R)))
    assert best * N == got["dev"]


def test_excesses_add_to_zero():
    for seed in range(20):
        text, image, _, _ = _tiny(seed)
        assert sum(packing.excess_numerators(text, image)) == 0


def test_one_rank_and_one_modality_have_no_excess():
    text, image = [5, 0, 7, 3], [2, 9, 0, 4]
    got = packing.best_packing(text, image, 1, 1000)
    assert got["dev"] == 0 and got["load"] == sum(text) + sum(image)
    for tt, ii in (([0, 0, 0], [3, 5, 8]), ([3, 5, 8], [0, 0, 0])):
        got = packing.best_packing(tt, ii, 2, 100)
        assert got["dev"] == 0 and got["load"] == 8   # {8} and {3, 5}


def test_permutation_and_scaling():
    text, image = [4, 0, 9, 2, 0], [3, 8, 0, 5, 6]
    base = packing.best_packing(text, image, 2, 40)
    perm = [3, 0, 4, 1, 2]
    pt = [text[i] for i in perm]
    pi = [image[i] for i in perm]
    assert (packing.best_packing(pt, pi, 2, 40)["dev"], packing.best_packing(pt, pi, 2, 40)["load"]) \
        == (base["dev"], base["load"])
    # counts times 3: N and V triple, so the numerators scale by 9 and the
    # token excess by 3
    sc = packing.best_packing([3 * t for t in text], [3 * v for v in image], 2, 120)
    assert sc["dev"] == 9 * base["dev"] and sc["load"] == 3 * base["load"]


def test_more_capacity_never_hurts():
    text, image = [7, 0, 5, 1, 3], [0, 6, 2, 6, 0]
    prev = None
    for cap in (14, 16, 20, 30):
        got = packing.best_packing(text, image, 2, cap)
        if got is None:
            continue
        if prev is not None:
            assert (got["dev"], got["load"]) <= prev
        prev = (got["dev"], got["load"])


def test_infeasible_is_none():
    assert packing.best_packing([10, 10, 10], [0, 0, 0], 2, 15) is None
