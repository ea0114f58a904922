"""Matching rules between a GPU selection and the oracle.

TEST INFRASTRUCTURE ONLY.

The rule asked of the indexer is literal: returned scores within 2e-3
relative of the oracle's (bf16 inputs, float32 accumulation), and top-k sets
identical except for keys whose oracle score lies within that tolerance of
the k-th score.  Ties go to the lower index, so outside that band the set is
bit-exact.

Scores: a returned (u, s_gpu) passes when
    |s_gpu - s(u)| <= max(RTOL * |s(u)|, E(u)),
with RTOL = 2e-3.  E(u) = FLOOR * (F(u) + A(u)), FLOOR = 2^-17, is the a priori
bound of float32 accumulation on this score: F(u) = sum_j |w_j| sum_i |q_ji
k_ui| bounds the terms of the head dot products (d <= 128 terms each, error
<= d * 2^-24 = 2^-17 of their magnitude, which is also what can flip max(0, .)
on a dot within rounding of zero) and A(u) = sum_j |w_j| max(0, q_j . k_u)
the terms of the weighted head sum (<= 128 terms).  E only exceeds the literal
tolerance where the signed heads cancel: |s(u)| < E(u) / 2e-3, which float32
accumulation cannot resolve to 2e-3 relative; there, and only there, E is the
fallback.  Without F the bound is FLOOR * A.

Selections: let K_t = min(k, |candidates|), O the oracle's top-K_t by (score
desc, index asc), s* the oracle's K_t-th score (E* its bound).  The tie band is
    band = {u : |s(u) - s*| <= max(RTOL * |s*|, E(u) + E*)}.
A GPU selection G passes when |G| = K_t, G has no duplicates, G is a subset of
the candidates, G minus band equals O minus band, and the k - K_t padding slots
hold (-1, -inf).

``stats`` (optional dict) counts what only the rounding fallback admitted:
"score_fallback" (scores outside the literal tolerance but within E) and
"band_fallback" (keys in the band only through E).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

RTOL = 2e-3
FLOOR = 2.0 ** -17


def rounding_bound(A: np.ndarray, F: Optional[np.ndarray]) -> np.ndarray:
    """E = FLOOR * (F + A): a priori float32 error bound of a score (F None: A only)."""
    A = np.asarray(A, dtype=np.float64)
    return FLOOR * (A if F is None else np.asarray(F, dtype=np.float64) + A)


def score_tolerance(s: np.ndarray, A: np.ndarray, F: Optional[np.ndarray],
                    rtol: float = RTOL) -> np.ndarray:
    """max(rtol * |s|, E): the literal relative tolerance, or the rounding bound
    where cancellation makes the literal one unreachable in float32."""
    return np.maximum(rtol * np.abs(np.asarray(s, dtype=np.float64)), rounding_bound(A, F))


def scores_ok(gpu: np.ndarray, s: np.ndarray, A: np.ndarray, F: Optional[np.ndarray] = None,
              rtol: float = RTOL, stats: Optional[Dict[str, int]] = None) -> np.ndarray:
    """Elementwise: GPU values within score_tolerance of the oracle's."""
    d = np.abs(np.asarray(gpu, dtype=np.float64) - np.asarray(s, dtype=np.float64))
    ok = d <= score_tolerance(s, A, F, rtol)
    if stats is not None:
        lit = d <= rtol * np.abs(np.asarray(s, dtype=np.float64))
        stats["score_fallback"] = stats.get("score_fallback", 0) + int((ok & ~lit).sum())
    return ok


def check_selection(gpu_idx: np.ndarray, gpu_val: Optional[np.ndarray], cand: np.ndarray,
                    s: np.ndarray, A: np.ndarray, k: int, F: Optional[np.ndarray] = None,
                    rtol: float = RTOL, what: str = "top-k",
                    stats: Optional[Dict[str, int]] = None) -> List[str]:
    """Check one query's selection.  ``cand``, ``s``, ``A``, ``F`` describe every
    candidate (ids and the oracle's scores over them).  Returns failure strings."""
    errs: List[str] = []
    cand = np.asarray(cand, dtype=np.int64)
    s = np.asarray(s, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    gpu_idx = np.asarray(gpu_idx).astype(np.int64)
    Kt = min(k, cand.size)
    G = gpu_idx[:Kt]
    pad = gpu_idx[Kt:]
    if np.any(pad != -1):
        errs.append(f"{what}: padding slots hold ids {pad[pad != -1][:8].tolist()}")
    if gpu_val is not None:
        pv = np.asarray(gpu_val, dtype=np.float64)[Kt:]
        if np.any(~(np.isneginf(pv))):
            errs.append(f"{what}: padding scores are not -inf")
    if np.unique(G).size != G.size:
        errs.append(f"{what}: duplicate ids in selection")
    pos_of = {int(u): i for i, u in enumerate(cand)}
    missing = [int(u) for u in G if int(u) not in pos_of]
    if missing:
        errs.append(f"{what}: ids outside the candidate set {missing[:8]}")
        return errs
    gi = np.array([pos_of[int(u)] for u in G], dtype=np.int64)
    Fg = None if F is None else np.asarray(F, dtype=np.float64)[gi]
    if gpu_val is not None and Kt:
        gv = np.asarray(gpu_val, dtype=np.float64)[:Kt]
        ok = scores_ok(gv, s[gi], A[gi], Fg, rtol, stats)
        if not np.all(ok):
            tol = score_tolerance(s[gi], A[gi], Fg, rtol)
            b = np.nonzero(~ok)[0][:4]
            errs.append(f"{what}: {int((~ok).sum())} scores off: " + ", ".join(
                f"u={int(G[i])} gpu={gv[i]!r} oracle={s[gi[i]]!r} tol={tol[i]:.3g}" for i in b))
    if Kt == 0:
        return errs
    order = np.lexsort((cand, -s))
    O = order[:Kt]
    s_star = s[O[-1]]
    E = rounding_bound(A, F)
    E_star = float(E[O[-1]])
    lit = np.abs(s - s_star) <= rtol * abs(s_star)
    band = lit | (np.abs(s - s_star) <= E + E_star)
    if stats is not None:
        stats["band_fallback"] = stats.get("band_fallback", 0) + int((band & ~lit).sum())
    g_out = set(int(x) for x in gi if not band[x])
    o_out = set(int(x) for x in O if not band[x])
    if g_out != o_out:
        extra = sorted(cand[list(g_out - o_out)].tolist())[:8]
        lost = sorted(cand[list(o_out - g_out)].tolist())[:8]
        errs.append(f"{what}: set differs outside the tie band (band size {int(band.sum())}); "
                    f"extra {extra} missing {lost}")
    return errs


def check_exact(gpu_idx: np.ndarray, ref_idx: np.ndarray, what: str = "selection") -> List[str]:
    """Bit-exact set equality of two padded selections (for exactly representable
    inputs where no tie band is needed)."""
    a = np.asarray(gpu_idx).astype(np.int64)
    b = np.asarray(ref_idx).astype(np.int64)
    if sorted(a.tolist()) != sorted(b.tolist()):
        return [f"{what}: {sorted(set(a.tolist()) ^ set(b.tolist()))[:8]} differ"]
    return []


def max_rel_err(gpu_val: np.ndarray, ref: np.ndarray, A: np.ndarray) -> float:
    """Largest |gpu - ref| / max(|ref|, A) over finite entries (for reports)."""
    g = np.asarray(gpu_val, dtype=np.float64)
    ok = np.isfinite(g)
    if not np.any(ok):
        return 0.0
    den = np.maximum(np.maximum(np.abs(ref[ok]), A[ok]), 1e-300)
    return float(np.max(np.abs(g[ok] - ref[ok]) / den))
