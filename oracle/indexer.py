"""Plain float64 NumPy oracle of the DSA indexer, MISA and HISA.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports this module.

Sources (page titles as printed; sections as they appear on each page):

* "MISA: Mixture of Indexer Sparse Attention for Long-Context LLM Inference"
  (technical summary).  Section "problem": the DSA indexer scores every prefix
  token through a pool of H_I heads and keeps the top-k tokens; cost O(H_I L).
  Section "method": blocks M = ceil(L/B), mean-pooled indexing keys, per-head
  affinity aggregated to a per-head importance, top-h heads, then only those h
  heads score the full prefix and the top-k is taken on the reduced scores.
  Section "hierarchical variant (MISA dagger)": the routed pass keeps k'
  candidates; all H_I heads rescore only those to give the final top-k.
* "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse Attention"
  (paper review).  Sections 1 and 3: split the prefix into blocks of size B,
  score pooled representative vectors, keep the top-m blocks, then score tokens
  only inside the surviving blocks and keep the top-k.
* "DoSA: Dots Sparse Attention" (paper review), sections 1 and 3: the indexer
  score is a multi-head relevance score whose heads are signed (negative
  contributions matter), and top-K selection picks exactly the K highest.
* The per-token score formula  s(t,u) = sum_j w[t,j] * max(0, q[t,j] . k[u])
  (no scale, no bias, no softmax) and the lower-index tie-break are the reading
  adopted for the method's own statement of the indexer; the pages print no
  formula.

Readings where the pages are silent (each also listed with the design notes):
  R1 score formula as above; R2 the prefix of query t is u = 0..pos_t
  inclusive; R3 one key per token shared by all heads; R5 pooling is the mean
  over the block's valid tokens, rounded once to bf16 (round-to-nearest-even);
  a partial last block is averaged over its valid tokens only; R6 MISA head
  importance I[t,j] = |w[t,j]| * sum_b max(0, q[t,j] . kbar[b]); ties to the
  lower head index; R7 routed heads keep their original weights; R8 HISA block
  score = the indexer formula with all heads applied to the pooled keys;
  R9 no forced sink/local blocks; R10 MISA dagger ranks candidates by the
  routed score and returns full H_I-head scores; R11 ties go to the lower
  index, output is a set padded with (-1, -inf), -0.0 equals +0.0; R18 the
  composition of the two (MISA summary, "method": the head axis; HISA review,
  section 3: the token axis) routes h heads with MISA's router and runs both
  HISA stages with only those heads, original weights kept.

Pins (what checks each function against something other than itself; the
tests live in tests/test_oracle_*.py):
  indexer_scores   hand-worked example (tests/golden), closed form with
                   axis-aligned vectors, H=1 reduces to max(0, q K^T) from a
                   library matmul, positive homogeneity, key permutation,
                   pure-Python brute force
  top_k            brute-force full sort, all-equal keys give 0..k-1,
                   short prefix returns all keys plus padding
  pool_block_bf16  constant block, B=1 identity, exact rounding cases on the
                   bf16 grid, brute force
  misa_*           h = H_I equals dense; brute force over all head subsets on
                   tiny H (the chosen set maximises the summed importance);
                   hand-worked example.  The importance formula itself (R6) is
                   "parity unpinned": the pages give no formula.
  misa_dagger      k' >= prefix equals dense; h = H_I equals dense
  hisa             m = M equals dense; B = 1 with m >= k equals dense;
                   hand-worked example.  The block-score formula (R8) is
                   "parity unpinned".
  misa_hisa        h = H_I equals HISA; m = M equals MISA; pure-Python brute
                   force.  The composition itself (R18) is a reading of the
                   pages, which name the combination but give no steps.
  dosa_*           the bounds bracket every score; the selection equals
                   dense_row's; h = H_I collapses both bounds onto the score
                   (survivors are exactly the keys at or above the k-th
                   score); brute force on tiny inputs.
  iou              hand-computed cases, IoU(A, A) = 1, disjoint = 0
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------- inputs ---

def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16) or float32 data."""
    if dtype == "bf16":
        b = np.ascontiguousarray(x).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------- scores ---

def head_dots(q_t: np.ndarray, K: np.ndarray) -> np.ndarray:
    """q_t [H, d] and K [n, d] -> the H x n matrix of head-key dot products."""
    return q_t @ K.T


def indexer_scores(q_t: np.ndarray, w_t: np.ndarray, K: np.ndarray
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Indexer score of every key in K for one query (R1), and its magnitude.

    s[u] = sum_j w[j] * max(0, q[j] . k[u]);  A[u] = sum_j |w[j]| * max(0, q[j] . k[u]).
    A >= |s| is the scale the matching tolerance is taken relative to.
    """
    R = np.maximum(head_dots(q_t, K), 0.0)
    return w_t @ R, np.abs(w_t) @ R


def dot_magnitude(q_t: np.ndarray, w_t: np.ndarray, K: np.ndarray) -> np.ndarray:
    """F[u] = sum_j |w[j]| * sum_i |q[j,i] k[u,i]|: the size of the terms a finite
    precision dot product accumulates; used only for the rounding floor of the
    matching tolerance."""
    return np.abs(w_t) @ (np.abs(q_t) @ np.abs(K).T)


# -------------------------------------------------------------- selection ---

def top_k(scores: np.ndarray, ids: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Exact top-k by (score descending, id ascending) (R11).

    Returns k ids and their scores; when fewer than k candidates exist the tail
    is padded with id -1 and score -inf.
    """
    scores = np.asarray(scores, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -scores))
    keep = order[:min(k, ids.size)]
    out_i = np.full(k, -1, dtype=np.int64)
    out_s = np.full(k, -np.inf, dtype=np.float64)
    out_i[:keep.size] = ids[keep]
    out_s[:keep.size] = scores[keep]
    return out_i, out_s


def prefix(pos: int) -> np.ndarray:
    """Causal prefix of a query at position pos: keys 0..pos inclusive (R2)."""
    return np.arange(int(pos) + 1, dtype=np.int64)


# ---------------------------------------------------------------- pooling ---

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even); returns the
    rounded values as float64.  bf16 keeps 8 significant bits; the spacing of
    the bf16 grid around |x| in [2^(e-1), 2^e) is 2^(e-8), and 2^-133 below the
    normal range."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(x / spacing) * spacing


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are already on the bf16 grid."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pool_block_bf16(K_block: np.ndarray) -> np.ndarray:
    """Mean of the block's keys (float64), rounded once to bf16 (R5)."""
    return round_bf16(K_block.mean(axis=0))


def pooled_keys(K_seq: np.ndarray, B: int, n_tokens: int) -> np.ndarray:
    """Pooled keys of the prefix keys 0..n_tokens-1: M = ceil(n_tokens / B) rows;
    block b covers tokens [b*B, min((b+1)*B, n_tokens)) (MISA "method" step 1;
    HISA section 3 stage 1)."""
    M = -(-int(n_tokens) // B)
    out = np.empty((M, K_seq.shape[1]), dtype=np.float64)
    for b in range(M):
        out[b] = pool_block_bf16(K_seq[b * B:min((b + 1) * B, n_tokens)])
    return out


def pooled_cache(K_seq: np.ndarray, B: int) -> np.ndarray:
    """Pooled keys of a whole key cache of l_max rows: ceil(l_max / B) blocks."""
    return pooled_keys(K_seq, B, K_seq.shape[0])


# ------------------------------------------------------------------ dense ---

def dense_row(q_t, w_t, K_seq, pos: int, k: int) -> Dict[str, np.ndarray]:
    """Dense DSA indexer for one query: score every prefix key, keep the top-k."""
    ids = prefix(pos)
    s, A = indexer_scores(q_t, w_t, K_seq[:pos + 1])
    idx, val = top_k(s, ids, k)
    return {"idx": idx, "val": val, "cand": ids, "s": s, "A": A}


# ------------------------------------------------------------------- MISA ---

def misa_importance(q_t, w_t, pooled: np.ndarray) -> np.ndarray:
    """Per-head importance from the pooled block keys (R6):
    I[j] = |w[j]| * sum_b max(0, q[j] . kbar[b])."""
    aff = np.maximum(head_dots(q_t, pooled), 0.0)   # [H, M] per-head affinity
    return np.abs(w_t) * aff.sum(axis=1)


def route_heads(I: np.ndarray, h: int) -> np.ndarray:
    """The h heads of largest importance, ties to the lower head index."""
    idx, _ = top_k(I, np.arange(I.size), h)
    return idx


def misa_pooled_for_query(K_seq, B: int, pos: int) -> np.ndarray:
    """Pooled keys visible to a query at pos: blocks of its own prefix."""
    return pooled_keys(K_seq, B, pos + 1)


def routed_scores(q_t, w_t, K_rows, heads: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Reduced score with only the routed heads (R7: original weights kept)."""
    hs = np.asarray(heads, dtype=np.int64)
    return indexer_scores(q_t[hs], w_t[hs], K_rows)


def misa_row(q_t, w_t, K_seq, pos: int, B: int, h: int, k: int,
             heads: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """MISA: route to h heads from pooled keys, score the full prefix with those
    heads, top-k on the reduced scores.  If ``heads`` is given, the routing step
    is skipped and that head set is used (for stage-conditional checks)."""
    pooled = misa_pooled_for_query(K_seq, B, pos)
    I = misa_importance(q_t, w_t, pooled)
    if heads is None:
        heads = route_heads(I, h)
    ids = prefix(pos)
    s, A = routed_scores(q_t, w_t, K_seq[:pos + 1], heads)
    idx, val = top_k(s, ids, k)
    return {"idx": idx, "val": val, "cand": ids, "s": s, "A": A, "I": I,
            "heads": np.asarray(heads), "pooled": pooled}


def rescore_row(q_t, w_t, K_seq, cand: np.ndarray, k: int) -> Dict[str, np.ndarray]:
    """Full H_I-head scores of a candidate set and its top-k (MISA dagger fine stage,
    HISA token-level refinement)."""
    cand = np.asarray(cand, dtype=np.int64)
    cand = cand[cand >= 0]
    s, A = indexer_scores(q_t, w_t, K_seq[cand])
    idx, val = top_k(s, cand, k)
    return {"idx": idx, "val": val, "cand": cand, "s": s, "A": A}


def misa_dagger_row(q_t, w_t, K_seq, pos: int, B: int, h: int, k_prime: int, k: int,
                    heads: Optional[np.ndarray] = None,
                    coarse: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """MISA dagger: the routed pass keeps k' candidates (coarse stage); all heads
    rescore them and the final top-k comes from the full scores (R10)."""
    m = misa_row(q_t, w_t, K_seq, pos, B, h, k_prime, heads=heads)
    if coarse is None:
        coarse = m["idx"]
    fine = rescore_row(q_t, w_t, K_seq, coarse, k)
    fine["coarse"] = m
    return fine


# ------------------------------------------------------------------- HISA ---

def hisa_block_scores(q_t, w_t, pooled: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Block scores from pooled keys with all heads (R8), and their magnitude."""
    return indexer_scores(q_t, w_t, pooled)


def hisa_candidates(blocks: np.ndarray, B: int, pos: int) -> np.ndarray:
    """Token positions of the surviving blocks, clipped to the causal prefix."""
    out: List[np.ndarray] = []
    for b in np.sort(np.asarray(blocks, dtype=np.int64)):
        if b < 0:
            continue
        out.append(np.arange(b * B, min((b + 1) * B, pos + 1), dtype=np.int64))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def hisa_row(q_t, w_t, K_seq, pos: int, B: int, m: int, k: int,
             blocks: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """HISA: keep the top-m blocks by pooled score, then score the tokens of the
    surviving blocks with all heads and keep the top-k.  If ``blocks`` is given,
    stage 1 is skipped and that block set is used."""
    pooled = misa_pooled_for_query(K_seq, B, pos)
    bs, bA = hisa_block_scores(q_t, w_t, pooled)
    if blocks is None:
        blocks, _ = top_k(bs, np.arange(pooled.shape[0]), m)
    cand = hisa_candidates(blocks, B, pos)
    fine = rescore_row(q_t, w_t, K_seq, cand, k)
    fine.update({"bs": bs, "bA": bA, "blocks": np.asarray(blocks), "pooled": pooled})
    return fine


# ------------------------------------------------- DoSA-style certificate ---

def dosa_certificate(q_t, w_t, K_rows, k: int, h: int) -> Dict[str, np.ndarray]:
    """A sound score certificate for exact top-k pruning (DoSA blog, sections
    1 and 3: screen with part of the heads, bound the rest, prune, rescore the
    survivors; the page gives no formulas, so these bounds are our own).
    Screening heads S: the h heads of largest |w_j| * ||q_j|| (ties to the
    lower index).  For every other head, Cauchy-Schwarz gives
    0 <= max(0, q_j . k) <= ||q_j|| * ||k||, so with s_S the exact screened sum
      LB(u) = s_S(u) + ||k_u|| * sum_{j not in S, w_j < 0} w_j ||q_j||
      UB(u) = s_S(u) + ||k_u|| * sum_{j not in S, w_j > 0} w_j ||q_j||
    bracket the full score.  The k keys of largest LB have true scores >= tau
    (the k-th largest LB), so the k-th largest score is >= tau and a key with
    UB < tau scores strictly below it: the exact top-k (ties included) lies
    among the survivors UB >= tau."""
    D = head_dots(q_t, K_rows)                         # [H, n]
    qn = np.sqrt((q_t * q_t).sum(axis=1))
    kn = np.sqrt((K_rows * K_rows).sum(axis=1))
    S, _ = top_k(np.abs(w_t) * qn, np.arange(w_t.size), h)
    rest = np.setdiff1d(np.arange(w_t.size), S)
    sS = w_t[S] @ np.maximum(D[S], 0.0)
    LB = sS + kn * (np.minimum(w_t[rest], 0.0) * qn[rest]).sum()
    UB = sS + kn * (np.maximum(w_t[rest], 0.0) * qn[rest]).sum()
    n = LB.size
    tau = np.sort(LB)[n - min(k, n)] if n else -np.inf
    return {"heads": S, "LB": LB, "UB": UB, "tau": tau, "survive": UB >= tau}


def dosa_row(q_t, w_t, K_seq, pos: int, k: int, h: int) -> Dict[str, np.ndarray]:
    """Exact top-k through the certificate: full scores for the survivors
    only, then their top-k; equals dense_row's selection."""
    ids = prefix(pos)
    c = dosa_certificate(q_t, w_t, K_seq[:pos + 1], k, h)
    keep = ids[c["survive"]]
    s, A = indexer_scores(q_t, w_t, K_seq[keep])
    idx, val = top_k(s, keep, k)
    return {"idx": idx, "val": val, "cand": keep, "s": s, "A": A, "cert": c}


# -------------------------------------------------------------- MISA∘HISA ---

def misa_hisa_row(q_t, w_t, K_seq, pos: int, B: int, h: int, m: int, k: int,
                  heads: Optional[np.ndarray] = None,
                  blocks: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """MISA∘HISA (R18): route to h heads from the pooled keys as MISA does,
    then run HISA with only those heads (original weights kept) in both of its
    stages: block scores over the pooled keys and token scores inside the kept
    blocks.  ``heads`` / ``blocks`` skip the routing / block stage (for
    stage-conditional checks)."""
    pooled = misa_pooled_for_query(K_seq, B, pos)
    I = misa_importance(q_t, w_t, pooled)
    if heads is None:
        heads = route_heads(I, h)
    hs = np.asarray(heads, dtype=np.int64)
    r = hisa_row(q_t[hs], w_t[hs], K_seq, pos, B, m, k, blocks=blocks)
    r.update({"I": I, "heads": hs})
    return r


# -------------------------------------------------------------------- IoU ---

def iou(a: np.ndarray, b: np.ndarray) -> float:
    """|A & B| / |A | B| over the non-padding indices; two empty sets give 1."""
    sa = set(int(x) for x in np.asarray(a).ravel() if x >= 0)
    sb = set(int(x) for x in np.asarray(b).ravel() if x >= 0)
    union = sa | sb
    if not union:
        return 1.0
    return len(sa & sb) / len(union)


def iou_rows(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Per-query IoU of two [nq, k] selections."""
    return np.array([iou(a, b) for a, b in zip(A, B)], dtype=np.float64)
