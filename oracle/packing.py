"""Token-count-aware packing across data-parallel ranks: the definition,
solved by exhaustive search on tiny inputs.

TEST INFRASTRUCTURE ONLY: the test suite may import this module; the
product (the HIP library's rvq_pack_ranks) never does, and shares no code
with it.

Source: "LongCat-2.5 Released", section 4 "Infrastructure: Under 80 GB Per
Card", "Supernode-aware parallelism", last paragraph; "LongCat-2.5 发布：面向
智能体任务的原生多模态大模型", "Supernode-Aware Parallelism", last paragraph.
Image-token counts are known when batches are packed, so the proportion of
visual tokens can be kept about the same on every data-parallel rank.  The
pages give that goal and no algorithm or objective; the reading taken here:

  sample i: t_i text tokens, v_i image tokens, n_i = t_i + v_i;
  batch: N = sum n_i, V = sum v_i, visual share p = V / N;
  an assignment puts every sample on one of R ranks, at most `capacity`
  tokens per rank; rank r then holds N_r tokens, V_r of them visual;
  objective: minimise D = max_r |V_r - p N_r|, then the largest load
  max_r N_r.

Everything is exact: N * (V_r - p N_r) = sum over the rank of
(v_i N - V n_i) is an integer, so the search compares integers.

Pins: tests/test_oracle_packing.py (hand-worked cases in
tests/golden/packing_hand_worked.json, closed forms, invariants, and the
objective recomputed in exact rationals).
"""
from __future__ import annotations

import itertools
from typing import Optional, Sequence


def excess_numerators(text: Sequence[int], image: Sequence[int]) -> list:
    """e_i = v_i N - V n_i: N times sample i's tokens beyond the batch's
    visual proportion (positive: more visual than the batch)."""
    N = sum(text) + sum(image)
    V = sum(image)
    return [v * N - V * (t + v) for t, v in zip(text, image)]


def evaluate(text, image, ranks: int, capacity: int, assignment) -> Optional[tuple]:
    """(max_r |N (V_r - p N_r)|, max_r N_r) of one assignment, or None when a
    rank holds more than `capacity` tokens."""
    e = excess_numerators(text, image)
    S = [0] * ranks
    load = [0] * ranks
    for i, r in enumerate(assignment):
        S[r] += e[i]
        load[r] += text[i] + image[i]
    if max(load) > capacity:
        return None
    return max(abs(s) for s in S), max(load)


def best_packing(text, image, ranks: int, capacity: int) -> Optional[dict]:
    """Every assignment of the samples to the ranks, the best kept: returns
    {"dev": max_r |N (V_r - p N_r)| (an integer), "N": N, "load": largest
    rank load, "optimal": every assignment reaching (dev, load)}, or None if
    no assignment fits the capacity.  Exponential: ranks ** samples."""
    best = None
    optimal = []
    for asg in itertools.product(range(ranks), repeat=len(text)):
        v = evaluate(text, image, ranks, capacity, asg)
        if v is None:
            continue
        if best is None or v < best:
            best, optimal = v, [asg]
        elif v == best:
            optimal.append(asg)
    if best is None:
        return None
    return {"dev": best[0], "N": sum(text) + sum(image), "load": best[1], "optimal": optimal}
