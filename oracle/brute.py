"""Pure-Python brute force of the indexer, MISA and HISA for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``indexer.py`` (no NumPy,
plain loops and ``sorted``) so that the two implementations pin each other on
tiny random inputs (H <= 4, d <= 8, L <= 64).  Inputs are nested Python lists
of floats (already-widened exact values).

Same definitions and readings as ``indexer.py``: score
sum_j w_j * max(0, q_j . k_u) over the inclusive causal prefix, exact top-k
ordered by (score descending, index ascending), mean-pooled blocks rounded to
bf16, MISA routing by |w_j| * sum_b max(0, q_j . kbar_b), HISA blocks by the
indexer score of the pooled keys.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import List, Sequence, Tuple


def dot(a: Sequence[float], b: Sequence[float]) -> float:
    total = 0.0
    for x, y in zip(a, b):
        total += x * y
    return total


def score(q_t: Sequence[Sequence[float]], w_t: Sequence[float], key: Sequence[float]) -> float:
    total = 0.0
    for j in range(len(w_t)):
        d = dot(q_t[j], key)
        if d > 0.0:
            total += w_t[j] * d
    return total


def select(pairs: List[Tuple[float, int]], k: int) -> List[int]:
    """pairs of (score, index): the k best by score desc, index asc; padded with -1."""
    ranked = sorted(pairs, key=lambda p: (-p[0], p[1]))
    out = [i for _, i in ranked[:k]]
    return out + [-1] * (k - len(out))


def dense(q_t, w_t, K, pos: int, k: int) -> List[int]:
    return select([(score(q_t, w_t, K[u]), u) for u in range(pos + 1)], k)


def bf16_round(x: float) -> float:
    """Nearest bf16 value, ties to even, by exact rational arithmetic."""
    if x == 0.0:
        return 0.0
    fx = Fraction(x)
    mag = abs(fx)
    e = math.floor(math.log2(mag))
    # correct e against floating error of log2
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    step = Fraction(2) ** max(e - 7, -133)
    n = fx / step
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(lo * step)


def pool(K, B: int, n_tokens: int) -> List[List[float]]:
    out = []
    for b in range((n_tokens + B - 1) // B):
        rows = K[b * B:min((b + 1) * B, n_tokens)]
        mean = [float(sum(Fraction(r[i]) for r in rows) / len(rows)) for i in range(len(K[0]))]
        out.append([bf16_round(v) for v in mean])
    return out


def importance(q_t, w_t, pooled) -> List[float]:
    out = []
    for j in range(len(w_t)):
        acc = 0.0
        for kb in pooled:
            d = dot(q_t[j], kb)
            if d > 0.0:
                acc += d
        out.append(abs(w_t[j]) * acc)
    return out


def misa(q_t, w_t, K, pos: int, B: int, h: int, k: int) -> Tuple[List[int], List[int]]:
    I = importance(q_t, w_t, pool(K, B, pos + 1))
    heads = select([(I[j], j) for j in range(len(I))], h)
    qh = [q_t[j] for j in heads]
    wh = [w_t[j] for j in heads]
    return heads, select([(score(qh, wh, K[u]), u) for u in range(pos + 1)], k)


def best_head_subset_value(I: Sequence[float], h: int) -> float:
    """Largest summed importance over all h-subsets of heads (exhaustive)."""
    return max(sum(I[j] for j in c) for c in itertools.combinations(range(len(I)), h))


def misa_dagger(q_t, w_t, K, pos: int, B: int, h: int, k_prime: int, k: int) -> List[int]:
    _, coarse = misa(q_t, w_t, K, pos, B, h, k_prime)
    return select([(score(q_t, w_t, K[u]), u) for u in coarse if u >= 0], k)


def hisa(q_t, w_t, K, pos: int, B: int, m: int, k: int) -> Tuple[List[int], List[int]]:
    pooled = pool(K, B, pos + 1)
    blocks = select([(score(q_t, w_t, pooled[b]), b) for b in range(len(pooled))], m)
    cand = []
    for b in blocks:
        if b >= 0:
            cand.extend(range(b * B, min((b + 1) * B, pos + 1)))
    return blocks, select([(score(q_t, w_t, K[u]), u) for u in cand], k)


def misa_hisa(q_t, w_t, K, pos: int, B: int, h: int, m: int, k: int):
    I = importance(q_t, w_t, pool(K, B, pos + 1))
    heads = select([(I[j], j) for j in range(len(I))], h)
    blocks, idx = hisa([q_t[j] for j in heads], [w_t[j] for j in heads], K, pos, B, m, k)
    return heads, blocks, idx


def iou(a: Sequence[int], b: Sequence[int]) -> float:
    sa = {x for x in a if x >= 0}
    sb = {x for x in b if x >= 0}
    if not (sa or sb):
        return 1.0
    return len(sa & sb) / len(sa | sb)


# ------------------------------------------- sparse attention over the list --

def sparse_mla(q_t: Sequence[Sequence[float]], rows: Sequence[Sequence[float]],
               idx_t: Sequence[int], d_v: int, scale: float) -> List[List[float]]:
    """Softmax attention of every head over the listed rows (entries outside
    the rows are skipped), value = the first d_v entries of each row; loops
    and math.exp only."""
    sel = [i for i in idx_t if 0 <= i < len(rows)]
    out = []
    for qh in q_t:
        if not sel:
            out.append([0.0] * d_v)
            continue
        s = [scale * dot(qh, rows[i]) for i in sel]
        top = max(s)
        e = [math.exp(x - top) for x in s]
        tot = sum(e)
        out.append([sum(e[n] * rows[sel[n]][c] for n in range(len(sel))) / tot
                    for c in range(d_v)])
    return out
