"""Exact-rational greedy RVQ for tiny inputs (pure Python, ``fractions``).

TEST INFRASTRUCTURE ONLY.  Used to pin the fp64 oracle's per-level choices
and gaps: every fp32 / fp64 input is a dyadic rational, so the distances,
argmins and residuals below carry no rounding at all.

Definition (greedy residual quantization, "LongCat-2.5 Open Source Release:
Meituan's 1.6T Multimodal Agent Model with 1M Context", section "02 Visual
Coding and 3D": detail is added level by level):
at each level the residual's squared Euclidean distance to every codeword of
that level's codebook is taken, the first index of the minimum is chosen,
the gap is the smallest distance over the other indices minus the minimum,
and the chosen codeword is subtracted.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple


def _frac_rows(a) -> List[List[Fraction]]:
    return [[Fraction(float(v)) for v in row] for row in a]


def encode_exact(x, codebooks) -> Tuple[List[List[int]], List[List[Fraction]]]:
    """Returns (ids[n][L], gaps[n][L]) with exact rational gaps
    (gap is None when a level has a single codeword)."""
    cb = [_frac_rows(level) for level in codebooks]
    ids_all, gaps_all = [], []
    for row in _frac_rows(x):
        r = list(row)
        ids, gaps = [], []
        for level in cb:
            dist = [sum((ri - ci) * (ri - ci) for ri, ci in zip(r, c)) for c in level]
            best = min(dist)
            k = dist.index(best)
            others = [v for j, v in enumerate(dist) if j != k]
            gaps.append(min(others) - best if others else None)
            ids.append(k)
            r = [ri - ci for ri, ci in zip(r, level[k])]
        ids_all.append(ids)
        gaps_all.append(gaps)
    return ids_all, gaps_all


def joint_exhaustive(x_row: Sequence[float], codebooks) -> Tuple[int, ...]:
    """Joint search: the ID tuple (one per level) minimising
    ||x - sum_l C_l[id_l]||^2 over all K^L tuples, first in lexicographic
    order on ties.  For tiny K and L only."""
    cb = [_frac_rows(level) for level in codebooks]
    x = [Fraction(float(v)) for v in x_row]
    L = len(cb)
    K = len(cb[0])
    best, best_t = None, None
    t = [0] * L
    while True:
        s = [xi for xi in x]
        for l in range(L):
            s = [si - ci for si, ci in zip(s, cb[l][t[l]])]
        v = sum(si * si for si in s)
        if best is None or v < best:
            best, best_t = v, tuple(t)
        l = L - 1
        while l >= 0:
            t[l] += 1
            if t[l] < K:
                break
            t[l] = 0
            l -= 1
        if l < 0:
            break
    return best_t
