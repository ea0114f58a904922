"""Python binding of libdsa_indexer.so, the gfx950 DSA indexer library.

Argument marshalling only: every step of the indexer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The C
contract (layouts, padding, error codes) is documented in include/dsa_indexer.h;
the functions here carry the same names.

If the shared library has not been built, every call raises; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

from ._abi import _SIGS, _i64  # ctypes signature table of the exported functions

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")

DSA_DTYPE_BF16 = 0
DSA_DTYPE_F32 = 1

# kernel kinds of dsa_kernel_timing_read
KERNEL_KINDS = {
    "prepare": 0, "score_tokens": 1, "score_pooled": 2, "score_list": 3, "score_blocks": 4,
    "route": 5, "pool": 6, "iou": 7, "prefill": 8, "rowselect": 9, "merge": 10,
    "route_heads": 11, "prefill_routed": 12, "hisa": 13, "mla": 14, "certify": 15,
}

_lib: Optional[ctypes.CDLL] = None


class DsaError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m sparse_attention_token_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().dsa_last_error().decode(errors="replace")
        raise DsaError(f"{what} failed (status {status}): {msg}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_DTYPE_BF16
    if t.dtype == torch.float32:
        return DSA_DTYPE_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16 or float32)")


def _need(t: torch.Tensor, name: str, dtype=None, dims=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")


def _workspace(nbytes: int, dev: torch.device, given: Optional[torch.Tensor]) -> torch.Tensor:
    if given is not None:
        _need(given, "workspace", torch.uint8, 1, dev)
        if given.numel() < nbytes or given.data_ptr() % 256:
            raise ValueError(f"workspace must hold >= {nbytes} bytes, 256-byte aligned")
        return given
    buf = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 1)]


def _common(q, w, k, q_pos, q_seq):
    _need(q, "q", dims=3)
    dev = q.device
    _need(w, "w", torch.float32, 2, dev)
    _need(k, "k", q.dtype, 3, dev)
    _need(q_pos, "q_pos", torch.int32, 1, dev)
    if q_seq is not None:
        _need(q_seq, "q_seq", torch.int32, 1, dev)
    nq, H, d = q.shape
    n_seq, l_max, dk = k.shape
    if w.shape != (nq, H) or dk != d or q_pos.shape[0] != nq or (
            q_seq is not None and q_seq.shape[0] != nq):
        raise ValueError("inconsistent shapes: q [nq,H,d], w [nq,H], k [n_seq,l_max,d], "
                         "q_pos/q_seq [nq]")
    return dev, nq, H, d, n_seq, l_max


def _status(dev, nq, out_status, with_status):
    if out_status is None:
        return torch.empty(nq, dtype=torch.int32, device=dev) if with_status else None
    _need(out_status, "out_status", torch.int32, 1, dev)
    if out_status.shape[0] != nq:
        raise ValueError("out_status must be [nq]")
    return out_status


def _outputs(dev, nq, k, out_idx, out_score, with_scores):
    if out_idx is None:
        out_idx = torch.empty((nq, k), dtype=torch.int32, device=dev)
    else:
        _need(out_idx, "out_idx", torch.int32, 2, dev)
        if tuple(out_idx.shape) != (nq, k):
            raise ValueError("out_idx must be [nq, top_k]")
    if out_score is None and with_scores:
        out_score = torch.empty((nq, k), dtype=torch.float32, device=dev)
    elif out_score is not None:
        _need(out_score, "out_score", torch.float32, 2, dev)
        if tuple(out_score.shape) != (nq, k):
            raise ValueError("out_score must be [nq, top_k]")
    return out_idx, out_score


def indexer_score_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max, top_k,
                                      dtype=DSA_DTYPE_BF16) -> int:
    return int(lib().indexer_score_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max,
                                                       top_k, dtype))


def indexer_score_topk(q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, q_pos: torch.Tensor,
                       q_seq: Optional[torch.Tensor] = None, top_k: int = 2048,
                       out_idx: Optional[torch.Tensor] = None,
                       out_score: Optional[torch.Tensor] = None, with_scores: bool = True,
                       workspace: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense DSA indexer: top_k prefix keys per query.  Returns (idx, scores)."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    dt = _dtype_code(q)
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    nbytes = indexer_score_topk_workspace_size(nq, H, d, n_seq, l_max, top_k, dt)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().indexer_score_topk(_ptr(q), _ptr(w), _ptr(k), dt, _ptr(q_seq), _ptr(q_pos), nq, H,
                                  d, n_seq, l_max, top_k, _ptr(out_idx), _ptr(out_score),
                                  _ptr(ws), nbytes, _stream(dev))
    _check(st, "indexer_score_topk")
    return out_idx, out_score


def indexer_score_topk_noalloc(q: torch.Tensor, w: torch.Tensor, k: torch.Tensor,
                               q_pos: torch.Tensor, q_seq: Optional[torch.Tensor] = None,
                               top_k: int = 2048, out_idx: Optional[torch.Tensor] = None,
                               out_score: Optional[torch.Tensor] = None, with_scores: bool = True
                               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The dense indexer on the library's own per-GPU scratch (no workspace;
    the C call allocates nothing).  Pass out_idx / out_score to allocate
    nothing here either.  Calls that overlap on one GPU race."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    dt = _dtype_code(q)
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    st = lib().indexer_score_topk_noalloc(_ptr(q), _ptr(w), _ptr(k), dt, _ptr(q_seq), _ptr(q_pos),
                                          nq, H, d, n_seq, l_max, top_k, _ptr(out_idx),
                                          _ptr(out_score), _stream(dev))
    _check(st, "indexer_score_topk_noalloc")
    return out_idx, out_score


NOALLOC_SCRATCH_BYTES = 80 << 20


def indexer_certified_topk_workspace_size(nq: int, n_heads: int, head_dim: int, n_seq: int,
                                          l_max: int, n_screen_heads: int, top_k: int) -> int:
    return int(lib().indexer_certified_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max,
                                                           n_screen_heads, top_k))


def indexer_certified_topk(q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, q_pos: torch.Tensor,
                           q_seq: Optional[torch.Tensor] = None, top_k: int = 2048,
                           n_screen_heads: int = 16, out_idx: Optional[torch.Tensor] = None,
                           out_score: Optional[torch.Tensor] = None, with_scores: bool = True,
                           with_survivors: bool = True, out_survivors: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Certified exact top-k (screened heads, Cauchy-Schwarz bounds for the
    others, survivors rescored with every head): the dense call's result.
    Returns {"idx", "score", "survivors"} (survivor count per query)."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    dt = _dtype_code(q)
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    surv = out_survivors
    if surv is None and with_survivors:
        surv = torch.empty(nq, dtype=torch.int32, device=dev)
    if surv is not None:
        _need(surv, "out_survivors", torch.int32, 1)
    nbytes = indexer_certified_topk_workspace_size(nq, H, d, n_seq, l_max, n_screen_heads, top_k)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().indexer_certified_topk(_ptr(q), _ptr(w), _ptr(k), dt, _ptr(q_seq), _ptr(q_pos), nq,
                                      H, d, n_seq, l_max, n_screen_heads, top_k, _ptr(out_idx),
                                      _ptr(out_score), _ptr(surv), _ptr(ws), nbytes, _stream(dev))
    _check(st, "indexer_certified_topk")
    out = {"idx": out_idx, "score": out_score}
    if surv is not None:
        out["survivors"] = surv
    return out


def indexer_mean_pool_keys(k: torch.Tensor, block: int,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean-pooled bf16 block keys [n_seq, ceil(l_max/block), d]."""
    _need(k, "k", torch.bfloat16, 3)
    n_seq, l_max, d = k.shape
    m = -(-l_max // block)
    if out is None:
        out = torch.empty((n_seq, m, d), dtype=torch.bfloat16, device=k.device)
    else:
        _need(out, "out", torch.bfloat16, 3, k.device)
        if tuple(out.shape) != (n_seq, m, d):
            raise ValueError("out must be [n_seq, ceil(l_max/block), d]")
    st = lib().indexer_mean_pool_keys(_ptr(k), DSA_DTYPE_BF16, n_seq, l_max, d, block, _ptr(out),
                                      _stream(k.device))
    _check(st, "indexer_mean_pool_keys")
    return out


def misa_route_score_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max, block,
                                         n_active_heads, k_prime, top_k, pooled_given) -> int:
    return int(lib().misa_route_score_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max,
                                                          block, n_active_heads, k_prime, top_k,
                                                          int(bool(pooled_given))))


def misa_route_score_topk(q, w, k, q_pos, q_seq=None, *, block: int, n_active_heads: int,
                          top_k: int, k_prime: int = 0, k_pooled=None, with_scores=True,
                          with_heads=True, with_importance=False, with_cand=False,
                          out_idx=None, out_score=None, workspace=None) -> Dict[str, torch.Tensor]:
    """MISA (k_prime == 0) or MISA dagger (k_prime >= top_k).  Returns a dict with
    "idx", "score" and, if asked, "heads", "importance", "cand"."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    if q.dtype != torch.bfloat16:
        raise TypeError("MISA takes bf16 inputs")
    if k_pooled is not None:
        _need(k_pooled, "k_pooled", torch.bfloat16, 3, dev)
        if tuple(k_pooled.shape) != (n_seq, -(-l_max // block), d):
            raise ValueError("k_pooled must be [n_seq, ceil(l_max/block), d]")
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    heads = torch.empty((nq, n_active_heads), dtype=torch.int32, device=dev) if with_heads else None
    imp = torch.empty((nq, H), dtype=torch.float32, device=dev) if with_importance else None
    cand = (torch.empty((nq, k_prime), dtype=torch.int32, device=dev)
            if (with_cand and k_prime > 0) else None)
    nbytes = misa_route_score_topk_workspace_size(nq, H, d, n_seq, l_max, block, n_active_heads,
                                                  k_prime, top_k, k_pooled is not None)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().misa_route_score_topk(_ptr(q), _ptr(w), _ptr(k), _ptr(k_pooled), DSA_DTYPE_BF16,
                                     _ptr(q_seq), _ptr(q_pos), nq, H, d, n_seq, l_max, block,
                                     n_active_heads, k_prime, top_k, _ptr(out_idx),
                                     _ptr(out_score), _ptr(heads), _ptr(imp), _ptr(cand), _ptr(ws),
                                     nbytes, _stream(dev))
    _check(st, "misa_route_score_topk")
    out = {"idx": out_idx, "score": out_score}
    if heads is not None:
        out["heads"] = heads
    if imp is not None:
        out["importance"] = imp
    if cand is not None:
        out["cand"] = cand
    return out


def hisa_block_filter_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max, block, m_blocks,
                                          top_k, pooled_given) -> int:
    return int(lib().hisa_block_filter_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max,
                                                           block, m_blocks, top_k,
                                                           int(bool(pooled_given))))


def hisa_block_filter_topk(q, w, k, q_pos, q_seq=None, *, block: int, m_blocks: int, top_k: int,
                           k_pooled=None, with_scores=True, with_blocks=True, with_status=True,
                           out_idx=None, out_score=None, out_status=None,
                           workspace=None) -> Dict[str, torch.Tensor]:
    """HISA: top-m pooled blocks, then top_k tokens inside them.  Returns a dict
    with "idx", "score" and, if asked, "blocks", "block_score" and "status"
    ([nq] int32: 1 where the query's wait for its block selection timed out and
    its row holds padding only; see dsa_hisa_wait_limit)."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    if q.dtype != torch.bfloat16:
        raise TypeError("HISA takes bf16 inputs")
    if k_pooled is not None:
        _need(k_pooled, "k_pooled", torch.bfloat16, 3, dev)
        if tuple(k_pooled.shape) != (n_seq, -(-l_max // block), d):
            raise ValueError("k_pooled must be [n_seq, ceil(l_max/block), d]")
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    blocks = torch.empty((nq, m_blocks), dtype=torch.int32, device=dev) if with_blocks else None
    bscore = torch.empty((nq, m_blocks), dtype=torch.float32, device=dev) if with_blocks else None
    status = _status(dev, nq, out_status, with_status)
    nbytes = hisa_block_filter_topk_workspace_size(nq, H, d, n_seq, l_max, block, m_blocks, top_k,
                                                   k_pooled is not None)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().hisa_block_filter_topk(_ptr(q), _ptr(w), _ptr(k), _ptr(k_pooled), DSA_DTYPE_BF16,
                                      _ptr(q_seq), _ptr(q_pos), nq, H, d, n_seq, l_max, block,
                                      m_blocks, top_k, _ptr(out_idx), _ptr(out_score),
                                      _ptr(blocks), _ptr(bscore), _ptr(status), _ptr(ws), nbytes,
                                      _stream(dev))
    _check(st, "hisa_block_filter_topk")
    out = {"idx": out_idx, "score": out_score}
    if blocks is not None:
        out["blocks"] = blocks
        out["block_score"] = bscore
    if status is not None:
        out["status"] = status
    return out


def misa_hisa_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max, block, n_active_heads,
                                  m_blocks, top_k, pooled_given) -> int:
    return int(lib().misa_hisa_topk_workspace_size(nq, n_heads, head_dim, n_seq, l_max, block,
                                                   n_active_heads, m_blocks, top_k,
                                                   int(bool(pooled_given))))


def misa_hisa_topk(q, w, k, q_pos, q_seq=None, *, block: int, n_active_heads: int,
                   m_blocks: int, top_k: int, k_pooled=None, with_scores=True, with_heads=True,
                   with_importance=False, with_blocks=True, with_status=True, out_idx=None,
                   out_score=None, out_status=None, workspace=None) -> Dict[str, torch.Tensor]:
    """MISA then HISA: h routed heads, then the top-m pooled blocks and the
    top_k tokens inside them, both scored with those heads.  Returns a dict
    with "idx", "score" and, if asked, "heads", "importance", "blocks",
    "block_score" and "status" (as for hisa_block_filter_topk)."""
    dev, nq, H, d, n_seq, l_max = _common(q, w, k, q_pos, q_seq)
    if q.dtype != torch.bfloat16:
        raise TypeError("MISA-HISA takes bf16 inputs")
    if k_pooled is not None:
        _need(k_pooled, "k_pooled", torch.bfloat16, 3, dev)
        if tuple(k_pooled.shape) != (n_seq, -(-l_max // block), d):
            raise ValueError("k_pooled must be [n_seq, ceil(l_max/block), d]")
    out_idx, out_score = _outputs(dev, nq, top_k, out_idx, out_score, with_scores)
    h = n_active_heads
    heads = torch.empty((nq, h), dtype=torch.int32, device=dev) if with_heads else None
    imp = torch.empty((nq, H), dtype=torch.float32, device=dev) if with_importance else None
    blocks = torch.empty((nq, m_blocks), dtype=torch.int32, device=dev) if with_blocks else None
    bscore = torch.empty((nq, m_blocks), dtype=torch.float32, device=dev) if with_blocks else None
    status = _status(dev, nq, out_status, with_status)
    nbytes = misa_hisa_topk_workspace_size(nq, H, d, n_seq, l_max, block, h, m_blocks, top_k,
                                           k_pooled is not None)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().misa_hisa_topk(_ptr(q), _ptr(w), _ptr(k), _ptr(k_pooled), DSA_DTYPE_BF16,
                              _ptr(q_seq), _ptr(q_pos), nq, H, d, n_seq, l_max, block, h,
                              m_blocks, top_k, _ptr(out_idx), _ptr(out_score), _ptr(heads),
                              _ptr(imp), _ptr(blocks), _ptr(bscore), _ptr(status), _ptr(ws),
                              nbytes, _stream(dev))
    _check(st, "misa_hisa_topk")
    out = {"idx": out_idx, "score": out_score}
    if heads is not None:
        out["heads"] = heads
    if imp is not None:
        out["importance"] = imp
    if blocks is not None:
        out["blocks"] = blocks
        out["block_score"] = bscore
    if status is not None:
        out["status"] = status
    return out


def hisa_wait_limit(ticks: int) -> None:
    """Bound of the HISA token pass's wait for its query's block selection, in
    ticks of the GPU's 100 MHz wall clock, for later calls; ticks < 0 restores
    the default (about 0.67 s).  For tests of the timeout path."""
    _check(lib().dsa_hisa_wait_limit(int(ticks)), "dsa_hisa_wait_limit")


def sparse_mla_workspace_size(nq, n_heads, d_qk, d_v, top_k) -> int:
    return int(lib().sparse_mla_workspace_size(nq, n_heads, d_qk, d_v, top_k))


def sparse_mla_attention(q, kv, q_pos, idx, q_seq=None, *, softmax_scale: float, out=None,
                         workspace=None) -> torch.Tensor:
    """Attention of every query's heads over the latent rows its index list
    names (absorbed-MLA form: q [nq, H, 576], kv [n_seq, L, 576], the first
    512 values of a row are its value).  Returns out [nq, H, 512] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(kv, "kv", torch.bfloat16, 3, dev)
    _need(q_pos, "q_pos", torch.int32, 1, dev)
    _need(idx, "idx", torch.int32, 2, dev)
    nq, H, d_qk = q.shape
    n_seq, l_max, d_kv = kv.shape
    if d_kv != d_qk:
        raise ValueError("q and kv rows must have the same width")
    if q_pos.shape[0] != nq or idx.shape[0] != nq:
        raise ValueError("q_pos and idx need one row per query")
    if q_seq is not None:
        _need(q_seq, "q_seq", torch.int32, 1, dev)
        if q_seq.shape[0] != nq:
            raise ValueError("q_seq needs one entry per query")
    top_k = idx.shape[1]
    d_v = 512
    if out is None:
        out = torch.empty((nq, H, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, 3, dev)
        if tuple(out.shape) != (nq, H, d_v):
            raise ValueError("out must be [nq, H, 512]")
    nbytes = sparse_mla_workspace_size(nq, H, d_qk, d_v, top_k)
    ws = _workspace(nbytes, dev, workspace)
    st = lib().sparse_mla_attention(_ptr(q), _ptr(kv), DSA_DTYPE_BF16, _ptr(q_seq), _ptr(q_pos),
                                    _ptr(idx), nq, H, d_qk, d_v, n_seq, l_max, top_k,
                                    float(softmax_scale), _ptr(out), _ptr(ws), nbytes,
                                    _stream(dev))
    _check(st, "sparse_mla_attention")
    return out


def indexer_selection_iou(a: torch.Tensor, b: torch.Tensor,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-row IoU of two [nq, k] int32 selections (padding -1 ignored)."""
    _need(a, "a", torch.int32, 2)
    _need(b, "b", torch.int32, 2, a.device)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    nq, k = a.shape
    if out is None:
        out = torch.empty(nq, dtype=torch.float32, device=a.device)
    st = lib().indexer_selection_iou(_ptr(a), _ptr(b), nq, k, _ptr(out), _stream(a.device))
    _check(st, "indexer_selection_iou")
    return out


def kernel_timing(enable: bool) -> None:
    """Record HIP events around every library kernel launch (measurement only)."""
    _check(lib().dsa_kernel_timing(int(bool(enable))), "dsa_kernel_timing")


def kernel_timing_read(kind: str) -> Dict[str, float]:
    """Launch count and summed / min / max duration (ms) of one kernel kind since
    the last read; waits for the recorded events."""
    n = _i64(0)
    tot, lo, hi = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _check(lib().dsa_kernel_timing_read(KERNEL_KINDS[kind], ctypes.byref(n), ctypes.byref(tot),
                                        ctypes.byref(lo), ctypes.byref(hi)),
           "dsa_kernel_timing_read")
    return {"launches": int(n.value), "total_ms": tot.value, "min_ms": lo.value,
            "max_ms": hi.value}


__all__ = [
    "kernel_timing", "kernel_timing_read", "KERNEL_KINDS",
    "DsaError", "LIB_PATH", "lib", "DSA_DTYPE_BF16", "DSA_DTYPE_F32",
    "indexer_score_topk", "indexer_score_topk_workspace_size", "indexer_score_topk_noalloc",
    "indexer_certified_topk", "indexer_certified_topk_workspace_size",
    "indexer_mean_pool_keys",
    "misa_route_score_topk", "misa_route_score_topk_workspace_size",
    "hisa_block_filter_topk", "hisa_block_filter_topk_workspace_size",
    "misa_hisa_topk", "misa_hisa_topk_workspace_size", "hisa_wait_limit",
    "sparse_mla_attention", "sparse_mla_workspace_size",
    "indexer_selection_iou",
]
