"""Pins of the screening oracle (oracle/rvq_screen.c), the encoder's codeword
decision emulated at the precision the encoder takes it in.  Each pin checks
it against something other than itself: torch's bf16 conversion, exact
rational arithmetic with the IEEE roundings written out, the fp64 oracle on
data where screening is exact, and hand-worked cases."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


# ---- exact rational model of the roundings (IEEE definitions) ----

def _round_bits(q: Fraction, p: int) -> Fraction:
    """q rounded to p significant bits, ties to even (normal range only)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scale = Fraction(2) ** (p - 1 - e)          # a * scale in [2^(p-1), 2^p)
    m = a * scale
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    out = Fraction(lo) / scale
    return out if q > 0 else -out


def _f32(q):
    return _round_bits(Fraction(q), 24)


def _bf16(q):
    return _round_bits(Fraction(q), 8)


def _chain(v):
    """Two fmaf chains over the halves (f & 8), each in increasing f, then
    one fp32 add; fmaf = exact a*b + c rounded once."""
    h = [Fraction(0), Fraction(0)]
    for f, vf in enumerate(v):
        b = (f >> 3) & 1
        h[b] = _f32(vf * vf + h[b])
    return _f32(h[0] + h[1])


def _exact_screen_encode(x, cb):
    """The decision procedure in exact rationals with explicit roundings:
    bf16 screening with the norm as bf16 hi + lo, the two smallest scores
    (lower index first) rescored in fp32, fp32 residual."""
    L, K, d = cb.shape
    ids = np.zeros((x.shape[0], L), dtype=np.int32)
    res = np.zeros(x.shape, dtype=np.float32)
    for row in range(x.shape[0]):
        r = [Fraction(float(v)) for v in x[row]]
        for l in range(L):
            br = [_bf16(v) for v in r]
            scores = []
            for k in range(K):
                c = [Fraction(float(v)) for v in cb[l, k]]
                nv = _chain(c)
                hi = _bf16(nv)
                lo = _bf16(nv - hi)
                s = hi + lo - 2 * sum(b * _bf16(cf) for b, cf in zip(br, c))
                scores.append((s, k))
            scores.sort()
            pair = [k for _, k in scores[:2]]
            if K == 1:
                win = 0
            else:
                dist = {k: _chain([_f32(rf - Fraction(float(cf))) for rf, cf in zip(r, cb[l, k])])
                        for k in pair}
                win = min(pair, key=lambda k: (dist[k], k))
            ids[row, l] = win
            r = [_f32(rf - Fraction(float(cf))) for rf, cf in zip(r, cb[l, win])]
        res[row] = np.array([float(v) for v in r], dtype=np.float32)
    return ids, res


# ---- pins ----

def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(11)
    v = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(100.0),
        g.standard_normal(2000).astype(np.float32) * np.float32(1e-3),
    ])
    # exact halfway cases, both parities of the kept last bit
    bits = (g.integers(0x3F000000, 0x43000000, 4000, dtype=np.uint32) & np.uint32(0xFFFF0000))
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, 1.0, -2.5, 65504.0])])
    got = oracle.screen_round_bf16(v)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(got.astype(np.float64), oracle.round_to_bf16(v))


def test_sq_chain_is_exact_on_small_integers():
    g = np.random.default_rng(12)
    v = g.integers(-40, 41, size=(64, 200)).astype(np.float32)
    got = oracle.screen_sq_chain(v)
    want = (v.astype(np.int64) ** 2).sum(axis=1)          # every partial sum < 2^24
    np.testing.assert_array_equal(got.astype(np.int64), want)


def test_sq_chain_equals_rational_fmaf_chains():
    g = np.random.default_rng(13)
    for d in (1, 7, 8, 9, 16, 17, 40, 71):
        v = g.standard_normal((6, d)).astype(np.float32)
        got = oracle.screen_sq_chain(v)
        for i in range(v.shape[0]):
            want = _chain([Fraction(float(t)) for t in v[i]])
            assert Fraction(float(got[i])) == want, (d, i)


def test_sq_chain_within_fp32_bound():
    g = np.random.default_rng(14)
    v = g.standard_normal((200, 1152)).astype(np.float32)
    got = oracle.screen_sq_chain(v).astype(np.float64)
    exact = (v.astype(np.float64) ** 2).sum(axis=1)
    n = 1152 // 2 + 1
    u = 2.0 ** -24
    assert np.all(np.abs(got - exact) <= n * u / (1 - n * u) * exact)


def _tiny_screen_problems():
    g = np.random.default_rng(15)
    out = []
    for (n, d, L, K) in [(4, 5, 3, 6), (3, 17, 2, 9), (2, 24, 3, 4), (3, 9, 2, 1), (2, 33, 2, 5)]:
        x = g.standard_normal((n, d)).astype(np.float32)
        cb = (g.standard_normal((L, K, d)) * 0.6).astype(np.float32)
        out.append((x, cb))
    # crowded codewords around one point, where which two are rescored
    # depends on rounding the residual to bf16 (seeds picked for that)
    for (seed, d, K, spread) in [(64, 2, 16, 0.01), (10, 1, 8, 0.02)]:
        g = np.random.default_rng(seed)
        base = g.standard_normal(d) * 4
        cb = (base + spread * g.standard_normal((1, K, d))).astype(np.float32)
        x = (base + spread * g.standard_normal((4, d))).astype(np.float32)
        out.append((x, cb))
    return out


N_TINY = 7


@pytest.mark.parametrize("case", range(N_TINY))
def test_matches_exact_rational_procedure(case):
    x, cb = _tiny_screen_problems()[case]
    ids, res = _exact_screen_encode(x, cb)
    out = oracle.screen_encode(x, cb)
    np.testing.assert_array_equal(out["ids"], ids)
    np.testing.assert_array_equal(out["res"].view(np.uint32), res.view(np.uint32))


def _exact_data(seed, n, d, L, K):
    """Halves in [-8, 8]: every bf16 copy, product, norm (with its hi + lo
    split) and residual is exact, so screening ranks exactly by distance."""
    g = np.random.default_rng(seed)
    x = (g.integers(-16, 17, size=(n, d)) / 2).astype(np.float32)
    cb = (g.integers(-16, 17, size=(L, K, d)) / 2).astype(np.float32)
    return x, cb


@pytest.mark.parametrize("seed,n,d,L,K", [(16, 60, 32, 3, 40), (17, 40, 20, 4, 7),
                                          (18, 30, 48, 2, 200)])
def test_equals_fp64_oracle_when_screening_is_exact(seed, n, d, L, K):
    x, cb = _exact_data(seed, n, d, L, K)
    out = oracle.screen_encode(x, cb)
    ref = oracle.encode(x, cb)
    np.testing.assert_array_equal(out["ids"], ref["ids"])
    np.testing.assert_array_equal(out["res"].astype(np.float64), ref["res"])


def test_hand_worked_screening_misses_the_nearest():
    # r = 1 + 2^-8 rounds to bf16 1.0 (a tie, to even).  Codewords
    # a = 1 + 2^-8 (distance 0), b = 1, c = 1 - 2^-8.  Scores hi + lo - 2 r c:
    #   a: (1 + 2^-7 + 2^-16) - 2 = -1 + 2^-7 + 2^-16
    #   b: 1 - 2 = -1
    #   c: (1 - 2^-7 + 2^-16) - 2 (1 - 2^-8) = -1 + 2^-16
    # so b and c are rescored: (2^-8)^2 < (2^-7)^2 and b wins, while the
    # exact nearest codeword is a.
    x = np.float32([[1 + 2 ** -8]])
    cb = np.float32([[[1 + 2 ** -8], [1.0], [1 - 2 ** -8]]])
    out = oracle.screen_encode(x, cb)
    assert out["ids"][0, 0] == 1 and out["n_options"][0, 0] == 1
    assert out["res"][0, 0] == np.float32(2 ** -8)
    assert oracle.encode(x, cb)["ids"][0, 0] == 0


def test_hand_worked_rescoring_overrides_screening():
    # a = 1 + 2^-9 and b = 1 + 2^-9 + 2^-11 both round to bf16 1.0, so the
    # screening ranks them by norm alone and puts a first; r = 1 + 2^-6 is
    # nearer to b, and rescoring picks b.
    x = np.float32([[1 + 2 ** -6]])
    cb = np.float32([[[1 + 2 ** -9], [1 + 2 ** -9 + 2 ** -11]]])
    out = oracle.screen_encode(x, cb)
    assert out["ids"][0, 0] == 1 and out["n_options"][0, 0] == 1
    assert oracle.encode(x, cb)["ids"][0, 0] == 1


def test_hand_worked_norm_low_part_decides():
    # Codewords 1 + e with e = 3, 1, 2 (units of 2^-12) all round to bf16
    # 1.0, and their norms 1 + 2e + e^2 all have bf16 high part 1.0, so only
    # the low part lo = bf16(2e + e^2) orders the scores: codewords 1 and 2
    # are rescored against r = 1 + 2^-8 (distances 15 and 14 units) and 2
    # wins.  The exact nearest is codeword 0 (13 units).
    x = np.float32([[1 + 2 ** -8]])
    cb = np.float32([[[1 + 3 * 2 ** -12], [1 + 2 ** -12], [1 + 2 * 2 ** -12]]])
    out = oracle.screen_encode(x, cb)
    assert out["ids"][0, 0] == 2 and out["n_options"][0, 0] == 1
    assert oracle.encode(x, cb)["ids"][0, 0] == 0


def test_near_equal_scores_admit_either_winner():
    # d = 1024, r = 1 + 2^-6 in every feature; codeword k = 1 + e_k in every
    # feature with e = 0, 2^-14, 2^-13, all rounding to bf16 1.0.  The scores
    # differ by the norms alone, about 2048 e_k apart (0.125 and 0.25), far
    # inside the bound on fp32 accumulation over 1024 products (about 0.4).
    # Unperturbed, codewords 0 and 1 are rescored and 1 wins; a GPU whose
    # sums rank 2 among the top two returns 2, the nearest.  0 never wins.
    d = 1024
    x = np.full((1, d), 1 + 2 ** -6, np.float32)
    cb = np.stack([np.full(d, 1 + e, np.float32) for e in (0.0, 2 ** -14, 2 ** -13)])[None]
    out = oracle.screen_encode(x, cb)
    assert out["ids"][0, 0] == 1 and out["n_options"][0, 0] == 2
    assert oracle.screen_encode(x, cb, follow=np.int32([[2]]))["admissible"][0, 0]
    assert not oracle.screen_encode(x, cb, follow=np.int32([[0]]))["admissible"][0, 0]
    assert oracle.encode(x, cb)["ids"][0, 0] == 2


def test_duplicated_codewords_tie_to_lowest_index():
    g = np.random.default_rng(19)
    cb = (g.standard_normal((2, 12, 16))).astype(np.float32)
    cb[:, 7] = cb[:, 3]
    cb[:, 9] = cb[:, 3]
    x = (cb[0, 3] + 0.01 * g.standard_normal((5, 16))).astype(np.float32)
    out = oracle.screen_encode(x, cb)
    assert np.all(out["ids"][:, 0] == 3)


def test_follow_own_choice_and_admissibility():
    g = np.random.default_rng(20)
    x = g.standard_normal((300, 96)).astype(np.float32)
    cb = (g.standard_normal((4, 300, 96)) * 0.5).astype(np.float32)
    own = oracle.screen_encode(x, cb)
    assert own["admissible"].all() and (own["n_options"] >= 1).all()
    again = oracle.screen_encode(x, cb, follow=own["ids"])
    assert again["admissible"].all()
    np.testing.assert_array_equal(again["n_options"], own["n_options"])
    np.testing.assert_array_equal(again["res"].view(np.uint32), own["res"].view(np.uint32))
    # the farthest codeword of level 0 is never admissible
    far = own["ids"].copy()
    r0 = x.astype(np.float64)
    dist = ((r0[:, None, :] - cb[0][None].astype(np.float64)) ** 2).sum(-1)
    far[:, 0] = dist.argmax(axis=1)
    bad = oracle.screen_encode(x, cb, follow=far)
    assert not bad["admissible"][:, 0].any()
    # nearly every decision is unique
    assert (own["n_options"] == 1).mean() > 0.99


def test_follow_rejects_out_of_range_ids():
    x = np.zeros((2, 8), np.float32)
    cb = np.ones((1, 3, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.screen_encode(x, cb, follow=np.int32([[0], [3]]))


def _rz32(v64):
    """fp64 -> fp32 rounded toward zero."""
    f = v64.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(v64)
    f[over] = np.nextafter(f[over], np.float32(0))
    return f


@pytest.mark.parametrize("d,K", [(1152, 48), (3, 300), (1, 400)])
def test_bound_covers_fp32_accumulation_orders(d, K):
    # The bound D on |key - S| must hold whatever order and rounding the
    # matrix cores use.  The terms of a score are exact in fp32 (hi, lo and
    # -2 bf16(r) bf16(c), at most 17 significant bits), so sum them in fp32
    # in several orders and with round-toward-zero, then replace the 5 low
    # mantissa bits by a tag at both extremes, as the ranking key does.
    # (At small d the tag bits, not the accumulation, dominate the bound.)
    g = np.random.default_rng(21 + d)
    r = g.standard_normal((6, d)).astype(np.float32)
    cb = g.standard_normal((K, d)).astype(np.float32)
    S, D = oracle.screen_scores(r, cb)
    br = oracle.screen_round_bf16(r).astype(np.float64)
    bc = oracle.screen_round_bf16(cb).astype(np.float64)
    nv = oracle.screen_sq_chain(cb)
    hi = oracle.screen_round_bf16(nv)
    lo = oracle.screen_round_bf16(nv - hi)
    worst = 0.0
    for i in range(r.shape[0]):
        for k in range(K):
            terms = np.concatenate([[hi[k], lo[k]], -2.0 * br[i] * bc[k]])
            t32 = terms.astype(np.float32)
            assert np.array_equal(t32.astype(np.float64), terms)
            sums = [np.add.accumulate(t32, dtype=np.float32)[-1],
                    np.add.accumulate(t32[::-1], dtype=np.float32)[-1],
                    np.sum(t32, dtype=np.float32)]
            acc = np.float32(hi[k] + lo[k])                  # one rounding per k-step of 16
            for j in range(2, len(terms), 16):
                acc = np.float32(np.float64(acc) + terms[j:j + 16].sum())
            sums.append(acc)
            acc = np.float32(0)                              # truncating adder
            for t in t32:
                acc = _rz32(np.array([np.float64(acc) + np.float64(t)]))[0]
            sums.append(acc)
            for v in sums:
                bits = np.float32(v).view(np.uint32)
                for tag in (0, 31):
                    key = np.uint32((bits & ~np.uint32(31)) | np.uint32(tag)).view(np.float32)
                    err = abs(float(key) - S[i, k])
                    assert err <= D[i, k], (i, k, err, D[i, k])
                    if D[i, k] > 0:
                        worst = max(worst, err / D[i, k])
    # the bound is a worst case, not a vacuous one
    assert 1e-4 < worst <= 1.0
    assert np.all(D < 1e-3 * (np.abs(S) + 4 * d))
