"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test names what it pins: the hand-worked fixture (tests/golden), closed
forms, special cases that reduce to a library routine, invariants, and the
independent pure-Python brute force.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import indexer as O
from oracle.check import check_selection

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


# ------------------------------------------------------ hand-worked example --

def test_hand_scores(gold):
    q, w, K = (np.array(gold[x], dtype=np.float64) for x in ("q", "w", "keys"))
    s, A = O.indexer_scores(q, w, K)
    assert s.tolist() == gold["scores"]
    assert A.tolist() == gold["magnitude"]
    for case in gold["dense"]:
        r = O.dense_row(q, w, K, case["pos"], case["k"])
        assert sorted(r["idx"].tolist()) == sorted(case["idx"])
        assert brute.dense(q.tolist(), w.tolist(), K.tolist(), case["pos"], case["k"]) \
            == case["idx"]


def test_hand_pool_misa_hisa(gold):
    q, w, K = (np.array(gold[x], dtype=np.float64) for x in ("q", "w", "keys"))
    assert O.pooled_keys(K, 2, 5).tolist() == gold["pooled_B2_pos4"]
    assert brute.pool(K.tolist(), 2, 5) == gold["pooled_B2_pos4"]
    m = gold["misa"]
    r = O.misa_row(q, w, K, m["pos"], m["B"], m["h"], m["k"])
    assert r["I"].tolist() == m["importance"]
    assert r["heads"].tolist() == m["heads"]
    assert r["idx"].tolist() == m["idx"]
    assert brute.misa(q.tolist(), w.tolist(), K.tolist(), m["pos"], m["B"], m["h"], m["k"]) \
        == (m["heads"], m["idx"])
    d = gold["misa_dagger"]
    r = O.misa_dagger_row(q, w, K, d["pos"], d["B"], d["h"], d["k_prime"], d["k"])
    assert sorted(r["coarse"]["idx"].tolist()) == sorted(d["coarse"])
    assert sorted(r["idx"].tolist()) == sorted(d["idx"])
    h = gold["hisa"]
    r = O.hisa_row(q, w, K, h["pos"], h["B"], h["m"], h["k"])
    assert r["bs"].tolist() == h["block_scores"]
    assert r["blocks"].tolist() == h["blocks"]
    assert sorted(r["idx"].tolist()) == sorted(h["idx"])
    assert brute.hisa(q.tolist(), w.tolist(), K.tolist(), h["pos"], h["B"], h["m"], h["k"]) \
        == (h["blocks"], h["idx"])
    dense3 = O.dense_row(q, w, K, 4, 3)["idx"]
    assert O.iou(r["idx"], dense3) == gold["iou_hisa_vs_dense_k3"]


# ------------------------------------------------------------- closed forms --

def test_closed_form_axis_aligned():
    """q_j = a_j e1, k_u = sigma_u e1: each dot is a_j sigma_u, so
    s_u = max(0, sigma_u) * sum_{a_j>0} w_j a_j + max(0, -sigma_u) * sum_{a_j<0} w_j |a_j|."""
    rng = np.random.default_rng(1)
    H, d, n = 6, 5, 40
    a = rng.standard_normal(H)
    w = rng.standard_normal(H)
    sig = rng.standard_normal(n)
    q = np.zeros((H, d)); q[:, 0] = a
    K = np.zeros((n, d)); K[:, 0] = sig
    s, A = O.indexer_scores(q, w, K)
    pos_part = np.sum(w[a > 0] * a[a > 0])
    neg_part = np.sum(w[a < 0] * -a[a < 0])
    expect = np.maximum(sig, 0) * pos_part + np.maximum(-sig, 0) * neg_part
    np.testing.assert_allclose(s, expect, rtol=1e-12, atol=1e-12)
    expect_A = np.maximum(sig, 0) * np.sum(np.abs(w[a > 0]) * a[a > 0]) + \
        np.maximum(-sig, 0) * np.sum(np.abs(w[a < 0]) * -a[a < 0])
    np.testing.assert_allclose(A, expect_A, rtol=1e-12, atol=1e-12)


def test_single_head_is_relu_matmul():
    """H = 1, w = 1: the score reduces to max(0, q . k), computed here by torch's
    CPU matrix-vector product and relu."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 16))
    K = rng.standard_normal((300, 16))
    s, A = O.indexer_scores(q, np.ones(1), K)
    ref = torch.relu(torch.mv(torch.from_numpy(K), torch.from_numpy(q[0]))).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(A, ref, rtol=1e-13, atol=1e-13)


def test_positive_homogeneity():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 8)); w = rng.standard_normal(4); K = rng.standard_normal((50, 8))
    s, _ = O.indexer_scores(q, w, K)
    s2, _ = O.indexer_scores(q, w, 4.0 * K)          # keys scaled by c > 0
    np.testing.assert_array_equal(s2, 4.0 * s)
    c = np.array([2.0, 0.5, 8.0, 0.25])               # q_j * c_j, w_j / c_j
    s3, _ = O.indexer_scores(q * c[:, None], w / c, K)
    np.testing.assert_allclose(s3, s, rtol=1e-13, atol=1e-13)
    s4, _ = O.indexer_scores(q, 2.0 * w, K)           # weights scaled
    np.testing.assert_array_equal(s4, 2.0 * s)


def test_key_permutation():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 8)); w = rng.standard_normal(3); K = rng.standard_normal((64, 8))
    perm = rng.permutation(64)
    s, _ = O.indexer_scores(q, w, K)
    sp, _ = O.indexer_scores(q, w, K[perm])
    np.testing.assert_allclose(sp, s[perm], rtol=1e-13, atol=1e-13)
    top, _ = O.top_k(s, np.arange(64), 10)
    topp, _ = O.top_k(sp, np.arange(64), 10)
    assert sorted(perm[topp].tolist()) == sorted(top.tolist())


# ------------------------------------------------------------------- top-k --

def test_topk_brute_force_sort_with_ties():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 80))
        k = int(rng.integers(1, 100))
        s = rng.integers(-5, 6, size=n).astype(np.float64)   # many exact ties
        ids = rng.permutation(1000)[:n]
        idx, val = O.top_k(s, ids, k)
        ranked = sorted(zip((-s).tolist(), ids.tolist()))[:k]
        expect = [i for _, i in ranked] + [-1] * (k - min(k, n))
        assert idx.tolist() == expect
        assert np.all(np.isneginf(val[min(k, n):]))


def test_topk_all_equal_gives_lowest_indices():
    idx, _ = O.top_k(np.zeros(500), np.arange(500), 64)
    assert idx.tolist() == list(range(64))
    # -0.0 and +0.0 are the same score
    s = np.where(np.arange(100) % 2 == 0, 0.0, -0.0)
    idx, _ = O.top_k(s, np.arange(100), 10)
    assert idx.tolist() == list(range(10))


def test_short_prefix_returns_all_and_pads():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 4)); w = rng.standard_normal(2); K = rng.standard_normal((10, 4))
    r = O.dense_row(q, w, K, 4, 8)
    assert sorted(r["idx"][:5].tolist()) == [0, 1, 2, 3, 4]
    assert r["idx"][5:].tolist() == [-1, -1, -1]
    assert np.all(np.isneginf(r["val"][5:]))


# ----------------------------------------------------------------- pooling --

def test_pool_special_cases():
    rng = np.random.default_rng(7)
    K = O.round_bf16(rng.standard_normal((64, 8)))
    np.testing.assert_array_equal(O.pooled_keys(K, 1, 64), K)            # B = 1
    const = np.tile(K[3], (16, 1))
    np.testing.assert_array_equal(O.pooled_keys(const, 16, 16), K[3:4])  # constant block
    np.testing.assert_array_equal(O.pooled_keys(K, 64, 64)[0], O.round_bf16(K.mean(axis=0)))


def test_bf16_rounding_exact_cases():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                        # tie -> even (mantissa 0)
        one + 3 * ulp / 2: one + 2 * ulp,          # tie -> even (mantissa 2)
        one + ulp / 2 + 2.0 ** -30: one + ulp,     # just above the tie
        -(one + ulp / 2): -one,
        3.0 * 2.0 ** -140: 2.0 ** -133 * 0.0 + 0.0,  # far below the smallest subnormal step
        2.0 ** -133 * 1.5: 2.0 ** -132,           # subnormal tie -> even
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.round_bf16(np.array([x]))[0] == want, x
        assert brute.bf16_round(x) == want, x


def test_pool_matches_brute_exact_rationals():
    rng = np.random.default_rng(8)
    for _ in range(20):
        L = int(rng.integers(1, 40)); B = int(rng.integers(1, 9)); d = 3
        K = O.round_bf16(rng.standard_normal((L, d)))
        n = int(rng.integers(1, L + 1))
        assert O.pooled_keys(K, B, n).tolist() == brute.pool(K.tolist(), B, n)


# -------------------------------------------------------- brute vs oracle --

def _int_inputs(rng, H, d, L):
    q = rng.integers(-3, 4, size=(H, d)).astype(np.float64)
    w = rng.integers(-4, 5, size=H).astype(np.float64) / 4.0
    K = rng.integers(-3, 4, size=(L, d)).astype(np.float64)
    return q, w, K


def test_dense_matches_brute_exact():
    rng = np.random.default_rng(9)
    for _ in range(60):
        H = int(rng.integers(1, 5)); d = int(rng.integers(1, 9)); L = int(rng.integers(1, 65))
        q, w, K = _int_inputs(rng, H, d, L)
        pos = int(rng.integers(0, L)); k = int(rng.integers(1, 20))
        r = O.dense_row(q, w, K, pos, k)
        assert r["idx"].tolist() == brute.dense(q.tolist(), w.tolist(), K.tolist(), pos, k)


def test_dense_matches_brute_float():
    rng = np.random.default_rng(10)
    for _ in range(30):
        H = int(rng.integers(1, 5)); d = int(rng.integers(1, 9)); L = int(rng.integers(1, 65))
        q = rng.standard_normal((H, d)); w = rng.standard_normal(H); K = rng.standard_normal((L, d))
        pos = int(rng.integers(0, L)); k = int(rng.integers(1, 20))
        r = O.dense_row(q, w, K, pos, k)
        b = brute.dense(q.tolist(), w.tolist(), K.tolist(), pos, k)
        assert check_selection(np.array(b), None, r["cand"], r["s"], r["A"], k) == []


def test_misa_hisa_match_brute_exact():
    rng = np.random.default_rng(11)
    for _ in range(40):
        H = int(rng.integers(1, 5)); d = int(rng.integers(1, 7)); L = int(rng.integers(2, 65))
        q, w, K = _int_inputs(rng, H, d, L)
        K = O.round_bf16(K)
        pos = int(rng.integers(0, L)); k = int(rng.integers(1, 20)); B = int(rng.integers(1, 9))
        h = int(rng.integers(1, H + 1))
        r = O.misa_row(q, w, K, pos, B, h, k)
        bh, bi = brute.misa(q.tolist(), w.tolist(), K.tolist(), pos, B, h, k)
        # integer inputs make importance ties common; the brute force resolves them
        # the same way (lower head index)
        assert r["heads"].tolist() == bh
        assert r["idx"].tolist() == bi
        kp = int(rng.integers(k, 40))
        rd = O.misa_dagger_row(q, w, K, pos, B, h, kp, k)
        assert sorted(rd["idx"].tolist()) == sorted(
            brute.misa_dagger(q.tolist(), w.tolist(), K.tolist(), pos, B, h, kp, k))
        m = int(rng.integers(1, 6))
        rh = O.hisa_row(q, w, K, pos, B, m, k)
        bb, bi = brute.hisa(q.tolist(), w.tolist(), K.tolist(), pos, B, m, k)
        assert rh["blocks"].tolist() == bb
        assert sorted(rh["idx"].tolist()) == sorted(bi)


def test_misa_hisa_matches_brute_and_reduces():
    """MISA∘HISA against the pure-Python composition on tiny integer inputs;
    with every head routed it is HISA, with every block kept it is MISA."""
    rng = np.random.default_rng(21)
    for _ in range(40):
        H = int(rng.integers(1, 5)); d = int(rng.integers(1, 7)); L = int(rng.integers(2, 65))
        q, w, K = _int_inputs(rng, H, d, L)
        K = O.round_bf16(K)
        pos = int(rng.integers(0, L)); k = int(rng.integers(1, 20)); B = int(rng.integers(1, 9))
        h = int(rng.integers(1, H + 1)); m = int(rng.integers(1, 6))
        r = O.misa_hisa_row(q, w, K, pos, B, h, m, k)
        bh, bb, bi = brute.misa_hisa(q.tolist(), w.tolist(), K.tolist(), pos, B, h, m, k)
        assert r["heads"].tolist() == bh
        assert r["blocks"].tolist() == bb
        assert sorted(r["idx"].tolist()) == sorted(bi)
        # every head routed: HISA (the head order does not change the sums'
        # exact integer values here)
        ra = O.misa_hisa_row(q, w, K, pos, B, H, m, k)
        rh = O.hisa_row(q, w, K, pos, B, m, k)
        assert sorted(ra["blocks"].tolist()) == sorted(rh["blocks"].tolist())
        assert sorted(ra["idx"].tolist()) == sorted(rh["idx"].tolist())
        # every block kept: MISA
        M = (pos + B) // B
        rm = O.misa_hisa_row(q, w, K, pos, B, h, M, k)
        mm = O.misa_row(q, w, K, pos, B, h, k)
        assert sorted(rm["idx"].tolist()) == sorted(mm["idx"].tolist())


def test_router_choice_maximises_importance():
    """Exhaustive search over all h-subsets of heads: the routed set attains the
    largest summed importance."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        H = int(rng.integers(2, 7)); h = int(rng.integers(1, H + 1))
        q = rng.standard_normal((H, 4)); w = rng.standard_normal(H)
        pooled = rng.standard_normal((9, 4))
        I = O.misa_importance(q, w, pooled)
        heads = O.route_heads(I, h)
        best = brute.best_head_subset_value(brute.importance(q.tolist(), w.tolist(),
                                                             pooled.tolist()), h)
        assert abs(I[heads].sum() - best) <= 1e-12 * max(1.0, best)


# -------------------------------------------------------------- invariants --

def test_misa_all_heads_equals_dense():
    rng = np.random.default_rng(13)
    q, w, K = _int_inputs(rng, 4, 6, 60)
    for pos in (0, 7, 59):
        for k in (1, 5, 70):
            d = O.dense_row(q, w, K, pos, k)
            m = O.misa_row(q, w, K, pos, 8, 4, k)
            assert sorted(m["idx"].tolist()) == sorted(d["idx"].tolist())
            md = O.misa_dagger_row(q, w, K, pos, 8, 2, 64, k)     # k' >= prefix
            assert sorted(md["idx"].tolist()) == sorted(d["idx"].tolist())
            md2 = O.misa_dagger_row(q, w, K, pos, 8, 4, k, k)     # h = H_I
            assert sorted(md2["idx"].tolist()) == sorted(d["idx"].tolist())


def test_hisa_all_blocks_or_unit_blocks_equals_dense():
    rng = np.random.default_rng(14)
    q, w, K = _int_inputs(rng, 3, 5, 50)
    for pos in (0, 13, 49):
        for k in (1, 6, 60):
            d = O.dense_row(q, w, K, pos, k)
            hm = O.hisa_row(q, w, K, pos, 8, 7, k)          # m = M (ceil(50/8) = 7)
            assert sorted(hm["idx"].tolist()) == sorted(d["idx"].tolist())
            h1 = O.hisa_row(q, w, K, pos, 1, max(k, 1), k)  # B = 1, m >= k
            assert sorted(h1["idx"].tolist()) == sorted(d["idx"].tolist())


def test_dot_magnitude_closed_form_and_loops():
    """F[u] = sum_j |w_j| sum_i |q_ji| |k_ui| (the term size behind the float32
    rounding bound of the matching rule): a hand-computed integer case, a loop
    over random integers, F >= A >= |s|, and planted mistakes that must differ
    (no |.| on q, on k or on w; a plain dot instead of the term-wise sum)."""
    q = np.array([[1.0, -2.0], [3.0, 0.0]])
    w = np.array([2.0, -1.0])
    K = np.array([[1.0, 1.0], [-2.0, 4.0]])
    # u=0: 2*(1*1 + 2*1) + 1*(3*1 + 0) = 9;  u=1: 2*(1*2 + 2*4) + 1*(3*2 + 0) = 26
    assert O.dot_magnitude(q, w, K).tolist() == [9.0, 26.0]
    rng = np.random.default_rng(21)
    caught = [False] * 4
    for _ in range(10):
        qq, ww, KK = _int_inputs(rng, 3, 4, 12)
        F = O.dot_magnitude(qq, ww, KK)
        loop = [sum(abs(ww[j]) * sum(abs(qq[j, i]) * abs(KK[u, i]) for i in range(qq.shape[1]))
                    for j in range(len(ww))) for u in range(len(KK))]
        assert F.tolist() == loop
        s, A = O.indexer_scores(qq, ww, KK)
        assert np.all(F >= A) and np.all(A >= np.abs(s))
        wrong = [np.abs(ww) @ np.abs(qq @ KK.T),               # |dot| instead of term-wise
                 np.abs(ww) @ (qq @ np.abs(KK).T),              # q without |.|
                 np.abs(ww) @ (np.abs(qq) @ KK.T),              # k without |.|
                 ww @ (np.abs(qq) @ np.abs(KK).T)]              # w without |.|
        for i, m in enumerate(wrong):
            caught[i] |= not np.array_equal(m, F)
    assert all(caught), caught
    # a planted mistake differs on the hand case too
    assert (np.abs(w) @ np.abs(q @ K.T)).tolist() != [9.0, 26.0]


def test_iou_cases():
    assert O.iou(np.array([1, 2, 3]), np.array([3, 2, 1])) == 1.0
    assert O.iou(np.array([1, 2]), np.array([3, 4])) == 0.0
    assert O.iou(np.array([1, 2, 3, -1]), np.array([2, 3, 4, 5])) == 2 / 5
    assert O.iou(np.array([-1, -1]), np.array([-1])) == 1.0
    assert brute.iou([1, 2, 3, -1], [2, 3, 4, 5]) == 2 / 5


# ---------------------------------------------- planted mistakes are caught --

def _mutants():
    def no_relu(q, w, K):
        D = q @ K.T
        return w @ D, np.abs(w) @ np.abs(D)

    def abs_weights(q, w, K):
        R = np.maximum(q @ K.T, 0)
        return np.abs(w) @ R, np.abs(w) @ R

    def relu_after_sum(q, w, K):
        s = w @ (q @ K.T)
        return np.maximum(s, 0), np.abs(s)

    def min_instead(q, w, K):
        R = np.minimum(q @ K.T, 0)
        return w @ R, np.abs(w) @ np.abs(R)

    def shifted_head(q, w, K):
        R = np.maximum(q @ K.T, 0)
        return np.roll(w, 1) @ R, np.abs(np.roll(w, 1)) @ R

    return [no_relu, abs_weights, relu_after_sum, min_instead, shifted_head]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_score_mistakes_fail_a_pin(mutant, gold):
    """Each plausible mistake in the score formula disagrees with the hand-worked
    example or with the brute force."""
    q, w, K = (np.array(gold[x], dtype=np.float64) for x in ("q", "w", "keys"))
    s, _ = mutant(q, w, K)
    caught = s.tolist() != gold["scores"]
    rng = np.random.default_rng(15)
    for _ in range(20):
        qq, ww, KK = _int_inputs(rng, 3, 4, 20)
        sm, _ = mutant(qq, ww, KK)
        sb = [brute.score(qq.tolist(), ww.tolist(), k) for k in KK.tolist()]
        caught |= not np.allclose(sm, sb)
    assert caught


def test_planted_selection_mistakes_fail_a_pin(gold):
    """Exclusive prefix, reversed tie-break and ascending order are all caught."""
    s = np.array(gold["scores"])
    want = gold["dense"][0]["idx"]
    assert sorted(np.lexsort((np.arange(4), -s[:4]))[:3].tolist()) != sorted(want)  # exclusive
    assert O.top_k(np.zeros(10), np.arange(10), 3)[0].tolist() == [0, 1, 2]
    assert np.lexsort((-np.arange(10), -np.zeros(10)))[:3].tolist() != [0, 1, 2]    # tie flip
    assert sorted(np.argsort(s)[:3].tolist()) != sorted(want)                         # ascending


# ------------------------------------------------- DoSA-style certificate ---

def _brute_certificate(q, w, K, k, h):
    """The certificate written out with loops: screening heads by |w_j| ||q_j||
    (ties to the lower index), exact screened sum, Cauchy-Schwarz for the rest."""
    import math
    H, n = len(w), len(K)
    qn = [math.sqrt(sum(x * x for x in q[j])) for j in range(H)]
    order = sorted(range(H), key=lambda j: (-abs(w[j]) * qn[j], j))
    S, rest = order[:h], order[h:]
    LB, UB = [], []
    for u in range(n):
        kn = math.sqrt(sum(x * x for x in K[u]))
        sS = sum(w[j] * max(0.0, sum(a * b for a, b in zip(q[j], K[u]))) for j in S)
        LB.append(sS + kn * sum(min(w[j], 0.0) * qn[j] for j in rest))
        UB.append(sS + kn * sum(max(w[j], 0.0) * qn[j] for j in rest))
    tau = sorted(LB)[n - min(k, n)]
    return sorted(S), LB, UB, tau


def test_dosa_certificate_brute_bounds_and_exact_selection():
    """The bounds against the loop form, bracketing every score; the pruned
    selection equals the dense one; with every head screened both bounds are
    the score and the survivors are exactly the keys at or above the k-th."""
    rng = np.random.default_rng(31)
    for it in range(60):
        H = int(rng.integers(1, 7)); d = int(rng.integers(1, 9)); L = int(rng.integers(1, 80))
        q = rng.standard_normal((H, d)); w = rng.standard_normal(H)
        K = rng.standard_normal((L, d))
        if it % 3 == 0:                              # a few keys along one head's query
            j = int(rng.integers(0, H))
            K[rng.integers(0, L, size=max(1, L // 8))] = q[j] + 0.3 * rng.standard_normal(d)
        pos = int(rng.integers(0, L)); k = int(rng.integers(1, 12)); h = int(rng.integers(1, H + 1))
        c = O.dosa_certificate(q, w, K[:pos + 1], k, h)
        S, LB, UB, tau = _brute_certificate(q.tolist(), w.tolist(), K[:pos + 1].tolist(), k, h)
        assert sorted(c["heads"].tolist()) == S
        assert np.allclose(c["LB"], LB, rtol=1e-12, atol=1e-12)
        assert np.allclose(c["UB"], UB, rtol=1e-12, atol=1e-12)
        s, _ = O.indexer_scores(q, w, K[:pos + 1])
        assert (c["LB"] <= s + 1e-9).all() and (s <= c["UB"] + 1e-9).all()
        r, dref = O.dosa_row(q, w, K, pos, k, h), O.dense_row(q, w, K, pos, k)
        assert sorted(r["idx"].tolist()) == sorted(dref["idx"].tolist())
    # integer inputs, every head screened: exact arithmetic, bounds = score
    for _ in range(20):
        H = int(rng.integers(1, 5)); d = int(rng.integers(1, 6)); L = int(rng.integers(2, 50))
        q, w, K = _int_inputs(rng, H, d, L)
        k = int(rng.integers(1, L + 1))
        c = O.dosa_certificate(q, w, K, k, H)
        s, _ = O.indexer_scores(q, w, K)
        assert np.array_equal(c["LB"], s) and np.array_equal(c["UB"], s)
        kth = np.sort(s)[L - k]
        assert np.array_equal(c["survive"], s >= kth)


@pytest.mark.parametrize("wid,row", [(2, 0), (3, 32767)])
def test_dosa_certificate_does_not_prune_the_synthetic_workloads(wid, row):
    """Measured, not a property of the method: on the dense decode and dense
    prefill inputs (Gaussian q, k in 128 dimensions) the Cauchy-Schwarz slack
    of the unscreened heads (about ||q|| ||k|| per head) dwarfs the spread of
    the scores, so even 48 of 64 screened heads leave over 90 % of the keys
    alive.  Exactness still holds."""
    import datagen
    wl = datagen.WORKLOADS[wid]
    q, w = datagen.queries(wl, 0)
    q_seq, q_pos = datagen.positions(wl)
    K = O.to_f64(datagen.keys(wl, int(q_seq[row]), q, w, 0), wl.dtype)
    q_t, w_t, pos = O.to_f64(q[row], wl.dtype), w[row].astype(np.float64), int(q_pos[row])
    for h in (16, 48):
        c = O.dosa_certificate(q_t, w_t, K[:pos + 1], wl.top_k, h)
        assert c["survive"].mean() > 0.9, (h, c["survive"].mean())
    r = O.dosa_row(q_t, w_t, K, pos, wl.top_k, 48)
    dref = O.dense_row(q_t, w_t, K, pos, wl.top_k)
    assert np.array_equal(np.sort(r["idx"]), np.sort(dref["idx"]))
