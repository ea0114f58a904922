"""CPU tests of the input generators and of the matching rules (fake backends)."""
import numpy as np

import datagen
from oracle import indexer as O
from oracle.check import FLOOR, RTOL, check_selection, rounding_bound, score_tolerance, scores_ok


def test_generation_is_deterministic_and_chunk_independent():
    wl = datagen.small(2, nq=3, n_seq=3, l_max=70000)
    q1, w1 = datagen.queries(wl, 0)
    q2, w2 = datagen.queries(wl, 0)
    assert np.array_equal(q1, q2) and np.array_equal(w1, w2)
    k_a = datagen.keys(wl, 1, q1, w1, 0)
    k_b = datagen.all_keys(wl, q1, w1, 0, threads=3)[1]
    assert np.array_equal(k_a, k_b)
    q3, _ = datagen.queries(wl, 1)
    assert not np.array_equal(q1, q3)


def test_bf16_rounding_of_generator():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    b = datagen.f32_to_bf16_bits(x)
    back = datagen.bf16_bits_to_f32(b)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]


def test_workload_shapes_and_positions():
    for wid, wl in datagen.WORKLOADS.items():
        seq, pos = datagen.positions(wl)
        assert seq.shape == (wl.nq,) and pos.shape == (wl.nq,)
        assert pos.max() < wl.l_max and pos.min() >= 0
        assert seq.max() < wl.n_seq
    seq, pos = datagen.positions(datagen.WORKLOADS[1])
    assert pos.tolist() == list(range(4080, 4096))


def test_planted_keys_follow_queries():
    wl = datagen.small(2, nq=2, n_seq=2, l_max=4096)
    q, w = datagen.queries(wl, 0)
    K = datagen.bf16_bits_to_f32(datagen.keys(wl, 0, q, w, 0)).astype(np.float64)
    qf = datagen.bf16_bits_to_f32(q).astype(np.float64)
    # a planted key correlates with one positive-weight head of its query
    cos = (K @ qf[0].T) / np.linalg.norm(K, axis=1)[:, None] / np.linalg.norm(qf[0], axis=1)
    assert (cos.max(axis=1) > 0.8).sum() == int(round(0.01 * 4096))


def _row(seed=0, n=300, H=4, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)); w = rng.standard_normal(H); K = rng.standard_normal((n, d))
    s, A = O.indexer_scores(q, w, K)
    F = O.dot_magnitude(q, w, K)
    return s, A, F


def test_checker_accepts_oracle_and_small_noise():
    s, A, F = _row()
    ids = np.arange(s.size)
    idx, val = O.top_k(s, ids, 20)
    assert check_selection(idx, val, ids, s, A, 20, F) == []
    perm = np.random.default_rng(1).permutation(20)
    noisy = val[perm] * (1 + 1e-5)
    assert check_selection(idx[perm], noisy, ids, s, A, 20, F) == []


def test_checker_rejects_wrong_sets_and_scores():
    s, A, F = _row()
    ids = np.arange(s.size)
    idx, val = O.top_k(s, ids, 20)
    order = np.lexsort((ids, -s))
    # swap a clear winner for a clear loser
    bad = idx.copy(); bad[0] = order[-1]
    assert check_selection(bad, None, ids, s, A, 20, F)
    # duplicate
    dup = idx.copy(); dup[1] = dup[0]
    assert check_selection(dup, None, ids, s, A, 20, F)
    # out of candidate set
    oob = idx.copy(); oob[2] = 10_000
    assert check_selection(oob, None, ids, s, A, 20, F)
    # score outside tolerance
    v = val.copy(); v[3] += 0.01 * max(abs(v[3]), A[idx[3]]) + 1.0
    assert check_selection(idx, v, ids, s, A, 20, F)
    # padding must be -1 / -inf
    short = np.arange(5)
    i5, v5 = O.top_k(s[:5], short, 8)
    assert check_selection(i5, v5, short, s[:5], A[:5], 8, F[:5]) == []
    i5b = i5.copy(); i5b[-1] = 0
    assert check_selection(i5b, v5, short, s[:5], A[:5], 8, F[:5])


def test_checker_tie_band_allows_swaps_only_inside_band():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-9, 1.0, 0.5])
    A = np.abs(s) + 1.0
    ids = np.arange(6)
    # oracle top-3 = {0, 1, 3}; 2 and 3 are within tolerance of each other
    assert check_selection(np.array([0, 1, 2]), None, ids, s, A, 3) == []
    assert check_selection(np.array([0, 1, 4]), None, ids, s, A, 3)
    # all-equal scores: every swap is inside the band, but the count must hold
    z = np.zeros(10)
    assert check_selection(np.array([9, 8, 7]), None, np.arange(10), z, z + 1, 3) == []


def _edge_row():
    """20 keys with distinct, well separated scores and no cancellation (A = |s|,
    F = 0): the rounding bound is 2^-17 |s|, far below the literal 2e-3 |s|."""
    s = 10.0 - 0.25 * np.arange(20)
    A = np.abs(s)
    F = np.zeros(20)
    return s, A, F


def test_checker_score_tolerance_edges():
    """A returned score 0.99x the tolerance away passes and 1.01x fails, in the
    literal regime (2e-3 relative) and in the cancellation regime, where the
    float32 rounding bound E = 2^-17 (F + A) is the tolerance."""
    s, A, F = _edge_row()
    ids = np.arange(20)
    idx, val = O.top_k(s, ids, 5)
    tol = RTOL * np.abs(val)
    for f, fails in ((0.99, False), (1.01, True)):
        for sign in (1.0, -1.0):
            v = val.copy()
            v[2] += sign * f * tol[2]
            assert bool(check_selection(idx, v, ids, s, A, 5, F)) == fails, (f, sign)
    # cancellation: a score of 1e-6 from terms of size 1 (A = 1, F = 10)
    s2 = np.array([3.0, 1e-6, -2.0])
    A2 = np.array([3.0, 1.0, 2.0])
    F2 = np.array([3.0, 10.0, 2.0])
    E = FLOOR * (F2[1] + A2[1])
    assert E > 100 * RTOL * s2[1]
    for f, fails in ((0.99, False), (1.01, True)):
        v = np.array([3.0, 1e-6 + f * E])
        assert bool(check_selection(np.array([0, 1]), v, np.arange(3), s2, A2, 2, F2)) == fails
    # the relative tolerance is not widened by the magnitude A any more: with
    # A = 2.2 |s| (typical cancellation at the k-th score), an error of
    # 1.5 x 2e-3 |s| fails although it is below 2e-3 A
    s3 = np.array([1.0, 0.5])
    A3 = np.array([2.2, 0.5])
    v3 = np.array([1.0 + 1.5 * RTOL])
    assert check_selection(np.array([0]), v3, np.arange(2), s3, A3, 1, np.zeros(2))


def test_checker_band_edge_swaps():
    """Swapping the k-th key for a key just inside the literal band (0.99 x
    2e-3 |s*| below s*) passes; just outside it (1.01 x) fails."""
    s, A, F = _edge_row()
    k = 5
    s_star = s[k - 1]
    ids = np.arange(20)
    for f, fails in ((0.99, False), (1.01, True)):
        s2 = s.copy()
        s2[k] = s_star - f * RTOL * abs(s_star)        # the next key, at the band edge
        A2 = np.abs(s2)
        idx, _ = O.top_k(s2, ids, k)
        swapped = idx.copy()
        swapped[k - 1] = k                              # k-th key out, edge key in
        assert bool(check_selection(swapped, None, ids, s2, A2, k, F)) == fails, f
        assert check_selection(idx, None, ids, s2, A2, k, F) == []


def test_checker_counts_what_only_the_rounding_bound_admits():
    s2 = np.array([3.0, 1e-6, -2.0])
    A2 = np.array([3.0, 1.0, 2.0])
    F2 = np.array([3.0, 10.0, 2.0])
    st = {}
    assert check_selection(np.array([0, 1]), np.array([3.0, 1e-6 + 1e-5]), np.arange(3), s2, A2,
                           2, F2, stats=st) == []
    assert st["score_fallback"] == 1
    st = {}
    s, A, F = _edge_row()
    assert check_selection(*O.top_k(s, np.arange(20), 5), np.arange(20), s, A, 5, F,
                           stats=st) == []
    assert st == {"score_fallback": 0, "band_fallback": 0}
    e = rounding_bound(A2, F2)
    assert np.allclose(score_tolerance(s2, A2, F2), np.maximum(RTOL * np.abs(s2), e))
    assert scores_ok(np.array([3.0 + 0.9 * RTOL * 3.0]), np.array([3.0]), np.array([3.0])).all()


def test_mla_inputs_regenerate_and_lists_are_valid():
    from datagen import mla as M
    wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"].replace(nq=6, n_seq=1, l_max=300,
                                                             n_heads=32, top_k=128, layout="tail")
    C = M.cache(wl, 3)
    pos = np.array([5, 299, 0, 17])
    assert np.array_equal(M.rows(wl, 0, pos, 3), C[0, pos])       # a row alone = in the cache
    assert not np.array_equal(M.rows(wl, 0, pos, 4), C[0, pos])   # the seed matters
    assert np.array_equal(M.queries(wl, 3), M.queries(wl, 3))
    _, qp = M.positions(wl)
    idx = M.index_lists(wl, 3)
    for t in range(wl.nq):
        n = int(qp[t]) + 1
        valid = idx[t][idx[t] >= 0]
        assert len(valid) == min(n, wl.top_k) and len(set(valid.tolist())) == len(valid)
        assert valid.max() < n and (idx[t][len(valid):] == -1).all()
    short = wl.replace(l_max=50, nq=3)                             # prefixes shorter than k
    li = M.index_lists(short, 1)
    assert (np.sort(li[0][li[0] >= 0]) == np.arange(48)).all() and (li[0][48:] == -1).all()
