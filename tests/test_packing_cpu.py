"""rvq_pack_ranks (the library's host-side packing planner, through its C
ABI) against the exhaustive packing oracle (oracle/packing.py)."""
import json
import os

import numpy as np
import pytest

from oracle import packing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing_hand_worked.json")


@pytest.fixture(scope="module")
def rvq():
    lib = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "residual_vector_quantization_rvq_amd", "librvq.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__._builder().build()
    import residual_vector_quantization_rvq_amd as m
    return m


def _check_summary(text, image, R, cap, ranks, summ):
    """The reported summary is the oracle's evaluation of the returned plan."""
    assert ranks.min() >= 0 and ranks.max() < R
    ev = packing.evaluate(text, image, R, cap, [int(r) for r in ranks])
    assert ev is not None, "plan exceeds the capacity"
    assert (summ["dev"], summ["max_load"]) == ev
    assert summ["N"] == sum(text) + sum(image)
    return ev


def _tiny(seed):
    g = np.random.default_rng(1000 + seed)
    S = int(g.integers(1, 9))
    R = int(g.integers(1, 4))
    text = [int(v) for v in g.integers(0, 40, S)]
    image = [int(v) if g.random() < 0.7 else 0 for v in g.integers(0, 40, S)]
    if sum(text) + sum(image) == 0:
        text[0] = 1
    cap = int(max(t + v for t, v in zip(text, image)) + g.integers(0, 80))
    return text, image, R, cap


@pytest.mark.parametrize("exact_max", [12, 0], ids=["exact", "heuristic"])
def test_hand_worked(rvq, exact_max):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ranks, summ = rvq.rvq_pack_ranks(c["text"], c["image"], c["ranks"], c["capacity"], exact_max)
        ev = _check_summary(c["text"], c["image"], c["ranks"], c["capacity"], ranks, summ)
        assert ev == (c["dev"], c["load"]), c["name"]


@pytest.mark.parametrize("seed", range(60))
def test_exact_mode_equals_the_oracle(rvq, seed):
    text, image, R, cap = _tiny(seed)
    want = packing.best_packing(text, image, R, cap)
    if want is None:
        with pytest.raises(rvq.RVQError):
            rvq.rvq_pack_ranks(text, image, R, cap, 12)
        return
    ranks, summ = rvq.rvq_pack_ranks(text, image, R, cap, 12)
    assert _check_summary(text, image, R, cap, ranks, summ) == (want["dev"], want["load"])


def test_heuristic_on_tiny_inputs(rvq):
    # greedy assignment plus improving moves and swaps: never more than one
    # sample's excess (max_i |e_i|) above the optimum; count how often it is
    # optimal
    equal = total = 0
    for seed in range(200):
        text, image, R, cap = _tiny(seed)
        want = packing.best_packing(text, image, R, cap)
        if want is None:
            continue
        try:
            ranks, summ = rvq.rvq_pack_ranks(text, image, R, cap, 0)
        except rvq.RVQError:
            continue  # the greedy may not find a fitting plan when the capacity is tight
        ev = _check_summary(text, image, R, cap, ranks, summ)
        e_max = max(abs(e) for e in packing.excess_numerators(text, image))
        assert ev[0] <= want["dev"] + e_max
        total += 1
        equal += ev[0] == want["dev"]
    print(f"[packing heuristic] optimal in {equal} of {total} tiny cases")
    assert total >= 100 and equal >= 0.8 * total


def _batch(seed, samples, text_only=0.3):
    """Samples of native-resolution image-text data: an image of H x W
    patches (H, W uniform on 14..84) after a text segment of 32..512
    tokens, or text alone (2,000..12,000 tokens) for a share of samples."""
    g = np.random.default_rng(seed)
    text = g.integers(32, 513, samples)
    image = g.integers(14, 85, samples) * g.integers(14, 85, samples)
    only = g.random(samples) < text_only
    text[only] = g.integers(2000, 12001, only.sum())
    image[only] = 0
    return text.astype(np.int64), image.astype(np.int64)


@pytest.mark.parametrize("samples,R", [(16, 2), (64, 4), (256, 8), (1024, 32)])
def test_heuristic_on_ragged_batches(rvq, samples, R):
    # one rank's modality excess stays below the largest single sample's,
    # and below 1% of the mean rank load once ranks hold several samples
    text, image = _batch(samples + R, samples)
    N = int(text.sum() + image.sum())
    cap = int(1.15 * N / R) + int((text + image).max())
    ranks, summ = rvq.rvq_pack_ranks(text, image, R, cap, 0)
    ev = _check_summary(list(map(int, text)), list(map(int, image)), R, cap, ranks, summ)
    e = packing.excess_numerators(list(map(int, text)), list(map(int, image)))
    dev_tokens = ev[0] / N
    print(f"[packing {samples} samples on {R} ranks] max excess {dev_tokens:.2f} tokens, "
          f"largest sample excess {max(map(abs, e)) / N:.1f}, mean load {N / R:.0f}")
    assert ev[0] <= max(abs(v) for v in e)
    if samples >= 8 * R:
        assert dev_tokens <= 0.01 * N / R


def test_arguments(rvq):
    with pytest.raises(rvq.RVQError):
        rvq.rvq_pack_ranks([5], [5], 0, 100)
    with pytest.raises(rvq.RVQError):
        rvq.rvq_pack_ranks([5, -1], [5, 1], 2, 100)
    with pytest.raises(rvq.RVQError):
        rvq.rvq_pack_ranks([50], [60], 2, 100)   # one sample above the capacity
    ranks, summ = rvq.rvq_pack_ranks([], [], 3, 10)
    assert ranks.shape == (0,) and summ["dev"] == 0
