"""Matching rules between a GPU selection and the oracle.

TEST INFRASTRUCTURE ONLY.

Scores: a returned (u, s_gpu) passes when
    |s_gpu - s(u)| <= RTOL * max(|s(u)|, A(u)) + FLOOR * F(u)
with RTOL = 2e-3 (bf16 inputs, fp32 accumulation), A(u) the sum of the absolute
head contributions (>= |s|, so the bound stays meaningful when signed heads
cancel), and F(u) = sum_j |w_j| sum_i |q_ji k_ui| times FLOOR = 2^-17 (= d * 2^-24
for d = 128): a bound on float32 accumulation rounding in the head dot products,
which is what can flip max(0, .) on a dot that is within rounding of zero.

Selections: let K_t = min(k, |candidates|), O the oracle's top-K_t by (score
desc, index asc), s* the oracle's K_t-th score.  The tie band is
    band = {u : |s(u) - s*| <= RTOL * max(|s*|, A(u)) + FLOOR * (F(u) + F*)}.
A GPU selection G passes when |G| = K_t, G has no duplicates, G is a subset of
the candidates, G minus band equals O minus band, and the k - K_t padding slots
hold (-1, -inf).  Outside the band the set is therefore bit-exact.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

RTOL = 2e-3
FLOOR = 2.0 ** -17


def _tol(s: np.ndarray, A: np.ndarray, F: Optional[np.ndarray], rtol: float) -> np.ndarray:
    t = rtol * np.maximum(np.abs(s), A)
    if F is not None:
        t = t + FLOOR * F
    return t


def check_selection(gpu_idx: np.ndarray, gpu_val: Optional[np.ndarray], cand: np.ndarray,
                    s: np.ndarray, A: np.ndarray, k: int, F: Optional[np.ndarray] = None,
                    rtol: float = RTOL, what: str = "top-k") -> List[str]:
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
    tol = _tol(s, A, F, rtol)
    if gpu_val is not None and Kt:
        gv = np.asarray(gpu_val, dtype=np.float64)[:Kt]
        bad = np.abs(gv - s[gi]) > tol[gi]
        if np.any(bad):
            b = np.nonzero(bad)[0][:4]
            errs.append(f"{what}: {int(bad.sum())} scores off: " + ", ".join(
                f"u={int(G[i])} gpu={gv[i]!r} oracle={s[gi[i]]!r} tol={tol[gi[i]]:.3g}" for i in b))
    if Kt == 0:
        return errs
    order = np.lexsort((cand, -s))
    O = order[:Kt]
    s_star = s[O[-1]]
    F_star = 0.0 if F is None else float(F[O[-1]])
    band_tol = rtol * np.maximum(abs(s_star), A)
    if F is not None:
        band_tol = band_tol + FLOOR * (F + F_star)
    band = np.abs(s - s_star) <= band_tol
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
