"""Pins for the fp64 oracle against facts fixed outside the oracle itself:
a hand-worked example, exact rational arithmetic, joint exhaustive search,
library routines (scipy's vector quantizer, torch's embedding bag, numpy's
bincount, torch's bf16 rounding), closed forms and invariants."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_2d.json")


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    cb = np.array(g["codebooks"], dtype=np.float32)
    x = np.array(g["x"], dtype=np.float32)
    return g, cb, x


def test_hand_worked_example_encode():
    g, cb, x = _golden()
    out = oracle.encode(x, cb)
    np.testing.assert_array_equal(out["ids"], np.array(g["ids"]))
    np.testing.assert_array_equal(out["gap"], np.array(g["gap"], dtype=np.float64))
    np.testing.assert_array_equal(out["rn2"], np.array(g["rn2"], dtype=np.float64))
    np.testing.assert_array_equal(out["ms"], np.array(g["ms"], dtype=np.float64))
    np.testing.assert_array_equal(out["res"], np.array(g["res"], dtype=np.float64))


def test_hand_worked_example_decode_hist_msr():
    g, cb, x = _golden()
    ids = np.array(g["ids"], dtype=np.int32)
    np.testing.assert_array_equal(oracle.decode(ids, cb), np.array(g["decode"], dtype=np.float64))
    np.testing.assert_array_equal(oracle.hist(ids, g["K"]), np.array(g["hist"]))
    np.testing.assert_array_equal(oracle.msr(x, ids, cb), np.array(g["msr"]))


def _tiny_problems():
    rng = np.random.default_rng(1234)
    for t in range(24):
        n = int(rng.integers(1, 7))
        d = int(rng.integers(1, 6))
        L = int(rng.integers(1, 4))
        K = int(rng.integers(1, 7))
        if t % 2 == 0:
            # small dyadic grid values: fp64 arithmetic on them is exact, and
            # exact distance ties happen often
            cb = (rng.integers(-4, 5, size=(L, K, d)) / 4.0).astype(np.float32)
            x = (rng.integers(-8, 9, size=(n, d)) / 4.0).astype(np.float32)
        else:
            cb = rng.standard_normal((L, K, d)).astype(np.float32)
            x = rng.standard_normal((n, d)).astype(np.float32)
        yield t, x, cb


@pytest.mark.parametrize("case", list(_tiny_problems()), ids=lambda c: f"t{c[0]}")
def test_matches_exact_rational_greedy(case):
    t, x, cb = case
    out = oracle.encode(x, cb)
    ids_e, gaps_e = exact.encode_exact(x, cb)
    np.testing.assert_array_equal(out["ids"], np.array(ids_e, dtype=np.int32).reshape(out["ids"].shape))
    for i in range(x.shape[0]):
        for l in range(cb.shape[0]):
            ge = gaps_e[i][l]
            if ge is None:
                assert math.isinf(out["gap"][i, l])
            elif t % 2 == 0:
                assert Fraction(out["gap"][i, l]) == ge
            else:
                assert abs(out["gap"][i, l] - float(ge)) <= 1e-12 * (1.0 + abs(float(ge)))


def test_duplicated_codewords_tie_to_lowest_index():
    rng = np.random.default_rng(7)
    d, K = 5, 6
    base = rng.standard_normal((K, d)).astype(np.float32)
    cb = np.stack([base, base]).copy()
    # duplicate codeword 4 into slots 1 and 5 of level 0 (so 1 is the lowest)
    cb[0, 1] = cb[0, 4]
    cb[0, 5] = cb[0, 4]
    x = (cb[0, 4] + np.float32(1e-3)).reshape(1, d)
    out = oracle.encode(x, cb)
    assert out["ids"][0, 0] == 1
    assert out["gap"][0, 0] == 0.0


def test_structured_rows_return_generating_ids():
    w = workloads.tiny_structured()
    half = w.N // 2
    out = oracle.encode(w.x, w.codebooks)
    np.testing.assert_array_equal(out["ids"][half:], w.gen_ids[half:])
    # certify each structured row: the tail sum of later levels is shorter
    # than half the distance from the true codeword to any other codeword
    # of its level, so the true codeword is the unique nearest (triangle
    # inequality); rounding x to fp32 moves it by far less than the margin.
    cb = w.codebooks.astype(np.float64)
    g = w.gen_ids[half:]
    for i in range(g.shape[0]):
        for l in range(w.L):
            tail = np.zeros(w.D)
            for j in range(l + 1, w.L):
                tail += cb[j, g[i, j]]
            sep = np.sqrt(((cb[l] - cb[l, g[i, l]]) ** 2).sum(axis=1))
            sep[g[i, l]] = np.inf
            assert np.linalg.norm(tail) < 0.5 * sep.min() - 1e-5
    # structured rows: strictly separated, final residual is fp32 rounding of x
    assert np.all(out["gap"][half:] > 1e-4 * out["rn2"][half:])
    assert np.abs(out["res"][half:]).max() < 1e-6


def test_greedy_equals_joint_search_on_separated_codebooks():
    rng = np.random.default_rng(11)
    L, K, d = 3, 4, 4
    cb = np.stack([(4.0 ** -l) * rng.standard_normal((K, d)) for l in range(L)]).astype(np.float32)
    gen = rng.integers(0, K, size=(6, L))
    x = np.stack([sum(cb[l, gen[i, l]].astype(np.float64) for l in range(L)) for i in range(6)]).astype(np.float32)
    out = oracle.encode(x, cb)
    for i in range(6):
        assert tuple(out["ids"][i]) == exact.joint_exhaustive(x[i], cb)


def test_is_greedy_not_joint():
    # 1-D case where greedy and joint search differ: greedy takes 3 at
    # level 0 (distance 1.96 < 2.56), then -2; joint prefers 0 then 2.
    cb = np.array([[[0.0], [3.0]], [[-2.0], [2.0]]], dtype=np.float32)
    x = np.array([[1.6]], dtype=np.float32)
    out = oracle.encode(x, cb)
    assert tuple(out["ids"][0]) == (1, 0)
    assert exact.joint_exhaustive(x[0], cb) == (0, 1)


def test_single_level_matches_scipy_vq():
    from scipy.cluster.vq import vq
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 16)).astype(np.float32)
    cb = rng.standard_normal((1, 37, 16)).astype(np.float32)
    out = oracle.encode(x, cb)
    code, dist = vq(x.astype(np.float64), cb[0].astype(np.float64))
    np.testing.assert_array_equal(out["ids"][:, 0], code)
    np.testing.assert_allclose(np.sqrt(out["ms"][:, 0]), dist, rtol=1e-12, atol=0)


def test_decode_matches_torch_embedding_bag():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    L, K, d, n = 5, 33, 24, 97
    cb = rng.standard_normal((L, K, d)).astype(np.float32)
    ids = rng.integers(0, K, size=(n, L)).astype(np.int32)
    table = torch.from_numpy(cb.astype(np.float64).reshape(L * K, d))
    flat = torch.from_numpy((ids + np.arange(L, dtype=np.int32) * K).reshape(-1).astype(np.int64))
    offs = torch.arange(0, n * L, L, dtype=torch.int64)
    ref = torch.nn.functional.embedding_bag(flat, table, offs, mode="sum").numpy()
    got = oracle.decode(ids, cb)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    # prefix decode with 0 levels is all zeros; with 1 level it is a lookup
    np.testing.assert_array_equal(oracle.decode(ids, cb, levels=0), np.zeros((n, d)))
    np.testing.assert_array_equal(oracle.decode(ids, cb, levels=1), cb[0][ids[:, 0]].astype(np.float64))


def test_embed_hand_worked_example():
    # level tables and a text table of small integers; the expected rows are
    # worked by hand: text -> the text row of ids[t, 0]; visual -> level-0 row
    # of ids[t, 0] plus level-1 row of ids[t, 1]
    vis = np.array([[[1, 2], [3, 4], [5, 6]], [[10, 20], [30, 40], [50, 60]]], dtype=np.float32)
    text = np.array([[100, 200], [300, 400]], dtype=np.float32)
    ids = np.array([[1, 0], [2, 0], [0, 2], [0, 2]], dtype=np.int32)
    flags = np.array([0, 1, 1, 0], dtype=np.uint8)
    want = np.array([[300, 400], [15, 26], [51, 62], [100, 200]], dtype=np.float64)
    np.testing.assert_array_equal(oracle.embed(ids, vis, flags, text), want)


def test_embed_visual_tokens_equal_decode():
    # a visual token's embedding is the decode of its IDs with the level
    # tables as codebooks (the decode is pinned against torch's embedding bag)
    rng = np.random.default_rng(10)
    L, K, D, T = 4, 19, 12, 50
    vis = rng.standard_normal((L, K, D)).astype(np.float32)
    ids = rng.integers(0, K, size=(T, L)).astype(np.int32)
    np.testing.assert_array_equal(oracle.embed(ids, vis), oracle.decode(ids, vis))
    np.testing.assert_array_equal(oracle.embed(ids, vis, np.ones(T, dtype=np.uint8)),
                                  oracle.decode(ids, vis))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embed_text_tokens_are_table_rows(dtype):
    rng = np.random.default_rng(11)
    L, K, D, V, T = 3, 7, 10, 23, 40
    vis = rng.standard_normal((L, K, D)).astype(np.float32)
    text = rng.standard_normal((V, D)).astype(np.float32)
    if dtype == "bf16":
        vis, text = workloads.bf16_bits_from_f32(vis), workloads.bf16_bits_from_f32(text)
    ids = rng.integers(0, K, size=(T, L)).astype(np.int32)
    flags = (rng.random(T) < 0.5).astype(np.uint8)
    ids[flags == 0, 0] = rng.integers(0, V, size=int((flags == 0).sum()))
    got = oracle.embed(ids, vis, flags, text, table_dtype=dtype)
    t64, v64 = oracle.as_f64(text, dtype), oracle.as_f64(vis, dtype)
    np.testing.assert_array_equal(got[flags == 0], t64[ids[flags == 0, 0]])
    vsum = sum(v64[l][ids[flags == 1, l]] for l in range(L))
    np.testing.assert_allclose(got[flags == 1], vsum, rtol=1e-15, atol=1e-15)


def test_residual_equals_input_minus_reconstruction():
    w = workloads.random_problem(21, n=40, d=48, L=6, K=64)
    out = oracle.encode(w.x, w.codebooks)
    recon = oracle.decode(out["ids"], w.codebooks)
    x64 = w.x.astype(np.float64)
    scale = np.abs(x64).sum(axis=1, keepdims=True) + np.abs(w.codebooks).max() * w.L
    assert np.all(np.abs(out["res"] - (x64 - recon)) <= 1e-12 * scale)
    # entering norm of level l+1 is the norm after level l; level 0 sees x
    np.testing.assert_array_equal(out["rn2"][:, 1:], out["ms"][:, :-1])
    np.testing.assert_allclose(out["rn2"][:, 0], (x64 * x64).sum(axis=1), rtol=1e-13)
    np.testing.assert_allclose(out["ms"][:, -1], (out["res"] ** 2).sum(axis=1), rtol=1e-13)
    assert np.all(out["gap"] >= 0)


def test_hist_matches_bincount():
    rng = np.random.default_rng(3)
    L, K, n = 4, 50, 1000
    ids = rng.integers(0, K, size=(n, L)).astype(np.int32)
    ids[::7] = 0
    h = oracle.hist(ids, K)
    for l in range(L):
        np.testing.assert_array_equal(h[l], np.bincount(ids[:, l], minlength=K))
    assert np.all(h.sum(axis=1) == n)
    with pytest.raises(ValueError):
        bad = ids.copy()
        bad[3, 2] = K
        oracle.hist(bad, K)


def test_msr_is_mean_squared_error_of_prefix_reconstruction():
    w = workloads.random_problem(22, n=30, d=20, L=4, K=16, x_dtype="bf16")
    out = oracle.encode(w.x, w.codebooks, x_dtype="bf16")
    m = oracle.msr(w.x, out["ids"], w.codebooks, x_dtype="bf16")
    x64 = oracle.widen_bf16(w.x).astype(np.float64)
    for l in range(w.L):
        rec = oracle.decode(out["ids"], w.codebooks, levels=l + 1)
        np.testing.assert_allclose(m[l], ((x64 - rec) ** 2).sum(axis=1).mean(), rtol=1e-12)
    np.testing.assert_allclose(m, out["ms"].mean(axis=0), rtol=1e-13)


def test_teacher_forced_excess():
    w = workloads.random_problem(23, n=12, d=8, L=3, K=10)
    out = oracle.encode(w.x, w.codebooks)
    tf = oracle.teacher_forced(w.x, out["ids"], w.codebooks)
    assert np.all(tf["excess"] == 0.0)
    np.testing.assert_array_equal(tf["rho2"], out["rn2"])
    # replace level-1 choices by the exact second-best: excess equals the gap
    ids2 = out["ids"].copy()
    cb = [[[Fraction(float(v)) for v in c] for c in lev] for lev in w.codebooks]
    for i in range(w.N):
        r = [Fraction(float(v)) for v in w.x[i]]
        r = [a - b for a, b in zip(r, cb[0][ids2[i, 0]])]
        dist = [sum((a - b) ** 2 for a, b in zip(r, c)) for c in cb[1]]
        order = sorted(range(w.K), key=lambda k: (dist[k], k))
        ids2[i, 1] = order[1]
    tf2 = oracle.teacher_forced(w.x, ids2, w.codebooks)
    np.testing.assert_allclose(tf2["excess"][:, 1], out["gap"][:, 1], rtol=1e-9, atol=1e-12)
    assert np.all(tf2["excess"][:, 0] == 0.0)


def test_round_to_bf16_single_rounding():
    torch = pytest.importorskip("torch")
    one = 1.0
    u = 2.0 ** -7  # bf16 spacing at 1
    cases = {
        one + u / 2: 1.0,                 # halfway, even neighbour is 1.0
        one + 1.5 * u: one + 2 * u,       # halfway, even neighbour is 1+2u
        one + u / 2 + 2.0 ** -30: one + u,  # just above halfway
        -3.0: -3.0,
        0.0: 0.0,
    }
    for v, want in cases.items():
        assert oracle.round_to_bf16(np.array([v]))[0] == want
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(20000) * 10.0).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(f.astype(np.float64)), ref)


def test_generators_are_deterministic_and_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    a = workloads.random_problem(5, n=64, d=32, L=2, K=8, x_dtype="bf16")
    b = workloads.random_problem(5, n=64, d=32, L=2, K=8, x_dtype="bf16")
    assert a.x.tobytes() == b.x.tobytes() and a.codebooks.tobytes() == b.codebooks.tobytes()
    f = workloads.random_problem(5, n=64, d=32, L=2, K=8, x_dtype="f32").x
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(a.x, ref)
    np.testing.assert_array_equal(oracle.widen_bf16(a.x), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_tiny_structured_workload_shape():
    w = workloads.tiny_structured()
    assert (w.N, w.D, w.L, w.K) == (256, 64, 4, 256)
    assert np.all(w.gen_ids[:128] == -1) and np.all(w.gen_ids[128:] >= 0)
    ratio = w.codebooks[0].std() / w.codebooks[1].std()
    assert 3.8 < ratio < 4.2


def test_single_image_rows_unit_norm():
    w = workloads.single_image()
    norms = np.linalg.norm(w.x.astype(np.float64), axis=1)
    assert np.all(np.abs(norms - 1.0) < 1e-6)
