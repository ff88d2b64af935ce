"""The encoder against the screening oracle (oracle/rvq_screen.c), which
takes each codeword decision the way the encoder's contract states it:
bf16 screening, the two best screened codewords rescored in fp32.  These
cases are chosen where that procedure and the exact nearest codeword part:
hand-worked inputs, and rows that randomised shape sweeps found."""
import numpy as np
import pytest
import torch

import oracle
import parity
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rvq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import residual_vector_quantization_rvq_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


# (name, row, codebook [K][d], screened ID, exact nearest); the derivations
# are in tests/test_oracle_screen.py
HAND = [
    ("screening_misses_the_nearest", [1 + 2 ** -8], [[1 + 2 ** -8], [1.0], [1 - 2 ** -8]], 1, 0),
    ("norm_low_part_decides", [1 + 2 ** -8],
     [[1 + 3 * 2 ** -12], [1 + 2 ** -12], [1 + 2 * 2 ** -12]], 2, 0),
    ("rescoring_overrides_screening", [1 + 2 ** -6], [[1 + 2 ** -9], [1 + 2 ** -9 + 2 ** -11]],
     1, 1),
]


@pytest.mark.parametrize("n", [1, 20000], ids=["split", "fused"])
@pytest.mark.parametrize("case", HAND, ids=lambda c: c[0])
def test_hand_worked_cases(rvq, dev, case, n):
    name, row, book, screened, nearest = case
    x = np.tile(np.float32(row), (n, 1))
    cb = np.float32(book)[None]
    assert oracle.encode(x[:1], cb)["ids"][0, 0] == nearest
    xd = torch.from_numpy(x).to(dev)
    cbd = torch.from_numpy(cb).to(dev)
    ids, res = rvq.rvq_encode(xd, cbd, rvq.rvq_prepare_codebooks(cbd), residual=True)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    print(f"[{name} n={n}] gpu {ids_h[0, 0]} screened {screened} nearest {nearest}")
    assert (ids_h == screened).all()
    parity.check_screened(x[:1], "f32", ids_h[:1], res.cpu().numpy()[:1], cb)


def test_near_equal_scores(rvq, dev):
    # codewords 1, 1 + 2^-14, 1 + 2^-13 at d = 1024 (all bf16 1.0): their
    # scores are closer than fp32 accumulation can resolve, so codeword 1 or
    # 2 may win; 0 may not
    d = 1024
    x = np.full((1, d), 1 + 2 ** -6, np.float32)
    cb = np.stack([np.full(d, 1 + e, np.float32) for e in (0.0, 2 ** -14, 2 ** -13)])[None]
    xd = torch.from_numpy(x).to(dev)
    cbd = torch.from_numpy(cb).to(dev)
    ids, res = rvq.rvq_encode(xd, cbd, rvq.rvq_prepare_codebooks(cbd), residual=True)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    print(f"[near_equal] gpu {ids_h[0, 0]}")
    assert ids_h[0, 0] in (1, 2)
    parity.check_screened(x, "f32", ids_h, res.cpu().numpy(), cb)


# Rows where the screening ranked the exact nearest codeword third, so the
# returned codeword is 1.1e-4 to 2.3e-4 ||r||^2 farther than the nearest:
# (seed, n, d, L, K, dtype, row, level, gap / ||r||^2 at least)
SWEEP_ROWS = [
    (1017, 23296, 50, 10, 3672, "f32", 16322, 3, 2.3e-4),
    (1027, 2350, 206, 11, 3721, "bf16", 561, 2, 1.3e-4),
    (1042, 1080, 450, 7, 1663, "bf16", 79, 0, 1.5e-4),
    (1004, 436, 149, 5, 4310, "f32", 100, 2, 1.5e-4),
    (1011, 21998, 1057, 5, 1712, "f32", 19741, 0, 1.1e-4),
]


@pytest.mark.parametrize("case", SWEEP_ROWS, ids=lambda c: f"s{c[0]}_d{c[2]}_row{c[6]}")
def test_sweep_rows_follow_the_screening(rvq, dev, case):
    seed, n, d, L, K, dt, row, level, rel = case
    w = workloads.random_problem(seed, n, d, L, K, x_dtype=dt)
    x = parity.x_to_device(w, dev)
    cb = torch.from_numpy(w.codebooks).to(dev)
    ids, res = rvq.rvq_encode(x, cb, rvq.rvq_prepare_codebooks(cb), residual=True)
    torch.cuda.synchronize()
    sel = np.array([0, row, n - 1])
    sub = w.rows(sel)
    ids_h = ids.cpu().numpy()[sel]
    res_h = res[torch.from_numpy(sel).to(dev)].cpu().numpy()
    stats = parity.check_screened(sub.x, dt, ids_h, res_h, w.codebooks)
    ref = oracle.encode(sub.x, sub.codebooks, x_dtype=dt)
    # the exact nearest path agrees up to the crowded level, where it parts
    np.testing.assert_array_equal(ids_h[1, :level], ref["ids"][1, :level])
    tf = oracle.teacher_forced(sub.x[1:2], ids_h[1:2], w.codebooks, x_dtype=dt)
    excess = tf["excess"][0, level] / tf["rho2"][0, level]
    own = oracle.screen_encode(sub.x[1:2], w.codebooks, x_dtype=dt)
    print(f"[sweep row s{seed}] gpu {ids_h[1]} nearest {ref['ids'][1]} screened {own['ids'][0]} "
          f"options {own['n_options'][0]} excess {excess:.3g} ||r||^2 screened {stats}")
    if own["n_options"][0, level] == 1:
        # a unique screened decision: the GPU takes it, not the nearest
        assert ids_h[1, level] == own["ids"][0, level] != ref["ids"][1, level]
        assert excess >= rel * 0.99
