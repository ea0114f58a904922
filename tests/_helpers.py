"""Helpers shared by the GPU parity tests: device upload of datagen inputs and
oracle runs over selected queries."""
from __future__ import annotations

import sys
from typing import Dict, Iterable, List, Optional

import numpy as np
import torch

import datagen
from oracle import indexer as O
from oracle.check import check_selection


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == datagen.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def upload(inp: Dict[str, np.ndarray], wl: datagen.Workload, dev="cuda") -> Dict[str, torch.Tensor]:
    return {
        "q": to_device(inp["q"], wl.dtype, dev),
        "w": torch.from_numpy(inp["w"]).to(dev),
        "k": to_device(inp["k"], wl.dtype, dev),
        "q_seq": torch.from_numpy(inp["q_seq"]).to(dev),
        "q_pos": torch.from_numpy(inp["q_pos"]).to(dev),
    }


def f64(inp: Dict[str, np.ndarray], wl: datagen.Workload, t: int):
    """Exact float64 q_t, w_t and the key cache of query t's sequence."""
    s = int(inp["q_seq"][t])
    return (O.to_f64(inp["q"][t], wl.dtype), inp["w"][t].astype(np.float64),
            O.to_f64(inp["k"][s], wl.dtype))


def check_rows(gi: np.ndarray, gv: Optional[np.ndarray], ref: Dict[int, dict], k: int,
               q_t_w_K: Dict[int, tuple], what: str = "top-k") -> List[str]:
    errs: List[str] = []
    for t, r in ref.items():
        q_t, w_t, K = q_t_w_K[t]
        cand = r["cand"]
        F = O.dot_magnitude(q_t, w_t, K[cand]) if cand.size else np.zeros(0)
        e = check_selection(gi[t], None if gv is None else gv[t], cand, r["s"], r["A"], k, F,
                            what=f"{what} q{t}")
        errs.extend(e)
    return errs


def dense_ref(inp, wl, rows: Iterable[int], k: int):
    ref, qwk = {}, {}
    for t in rows:
        q_t, w_t, K = f64(inp, wl, t)
        qwk[t] = (q_t, w_t, K)
        ref[t] = O.dense_row(q_t, w_t, K, int(inp["q_pos"][t]), k)
    return ref, qwk
