#!/usr/bin/env python3
"""Benchmark of the DSA indexer on one MI355X.

Default: the dense decode-shaped indexer, 64 queries each against its own
131072-key causal prefix, 64 heads, d = 128, bf16, top-k 2048.  One step = one
indexer_score_topk call (scoring and exact top-k selection of all 64 queries)
with inputs resident in HBM.  Prints one JSON line.

Other workloads (--workload): tiny (float32, 16 queries, L = 4096),
dense_prefill (32768 causal rows of one 32768-key cache), misa_prefill (the same
rows routed to h = 8 of 64 heads over 64-key pooled blocks), misa / misa_dagger
(h = 8 of 64 heads, B = 64, k' = 8192), hisa (32 heads, L = 1M, B = 128,
m = 64; --l-max shortens the caches and, at 128K or less, also times the
dense indexer on the same inputs), misa_hisa (the same with the router's
h = 8 heads), pool (mean
pooling of the 128K caches), sparse_mla (the attention that consumes the
index lists: 64 queries x 128 heads over 2048 listed rows of their own
131072-row latent caches, absorbed-MLA rows of 576 bf16 values),
dense_shared_decode (the 64 decode queries on one shared 131072-key cache),
certified (the certified exact top-k on the dense decode inputs: 16 screened
heads, bounds for the rest, survivors rescored; also times the dense call on
the same inputs).  tiny, hisa,
misa_hisa and sparse_mla touch less than the 256 MB last-level cache and are
timed cold.

The steps are timed twice: first the calls alone (ms_per_step, value), then
the same number of calls with the library's per-launch HIP events on the
call's stream, which give each kernel's average duration for the roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "sparse_attention_token_indexer_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOADS = {"dense_decode": 2, "tiny": 1, "dense_prefill": 3, "misa": 4, "misa_dagger": 4,
             "dense_shared_decode": 2, "certified": 2,
             "hisa": 5, "pool": 4, "misa_prefill": 3, "hisa_prefill": 3, "misa_hisa": 5,
             "sparse_mla": None}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
# the IoU against the dense indexer is measured up to this cache length (the
# dense call over the HISA workload's 1M-key caches is covered by the tests)
DENSE_IOU_MAX_L = 131072


# source file of each workload's dominant kernel (its hash, with every shared
# header's, identifies the build that traffic counters were taken on)
KERNEL_SOURCE = {"dense_decode": "k_score_select.hip", "tiny": "k_score_select.hip",
                 "misa": "k_score_select.hip", "misa_dagger": "k_score_select.hip",
                 "hisa": "k_hisa.hip", "dense_prefill": "k_prefill.hip",
                 "dense_shared_decode": "k_prefill.hip", "certified": "k_score_select.hip",
                 "misa_prefill": "k_prefill_routed.hip", "pool": "k_pool.hip",
                 "hisa_prefill": "k_hisa.hip", "misa_hisa": "k_hisa.hip",
                 "sparse_mla": "k_mla.hip"}


def _local_sources(name: str) -> list:
    """The source file and every header under csrc/ it includes, transitively."""
    seen, todo = [], [name]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.append(f)
        with open(os.path.join(CSRC, f)) as fh:
            for line in fh:
                line = line.strip()
                if line.startswith('#include "'):
                    todo.append(line.split('"')[1])
    return sorted(seen)


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in _local_sources(KERNEL_SOURCE[workload]):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from rocprofv3 counters, if they
    were taken on the current source of that kernel and the shared headers
    (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_hash") != kernel_source_hash(workload):
        return None
    return e.get("bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def gen_inputs(wl, seed, dev):
    import numpy as np
    import torch

    import datagen
    q, w = datagen.queries(wl, seed)
    q_seq, q_pos = datagen.positions(wl)

    def to_dev(x):
        if wl.dtype == datagen.BF16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    kdev = torch.empty((wl.n_seq, wl.l_max, wl.head_dim),
                       dtype=torch.bfloat16 if wl.dtype == datagen.BF16 else torch.float32, device=dev)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=16) as ex:
        for s, ks in enumerate(ex.map(lambda s: datagen.keys(wl, s, q, w, seed), range(wl.n_seq))):
            kdev[s].copy_(to_dev(ks))
    return {"q": to_dev(q), "w": torch.from_numpy(w).to(dev), "k": kdev,
            "q_seq": torch.from_numpy(q_seq).to(dev), "q_pos": torch.from_numpy(q_pos).to(dev),
            "np": {"q": q, "w": w, "q_seq": q_seq, "q_pos": q_pos}}


def cpu_baseline(wl, seed, seconds: float, mode: str):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole queries (full prefix scoring + exact top-k) until about `seconds` of
    compute have run.  Input generation is not timed."""
    import numpy as np

    import datagen
    from oracle import indexer as O
    q, w = datagen.queries(wl, seed)
    q_seq, q_pos = datagen.positions(wl)
    done_pairs, spent, nq_done = 0, 0.0, 0
    order = range(wl.nq)
    cache = {}
    if mode in ("dense_prefill", "misa_prefill", "hisa_prefill"):   # rows spread over the triangle
        order = np.random.default_rng(seed).permutation(wl.nq)
    for t in order:
        s_id = int(q_seq[t])
        if s_id not in cache:
            cache.clear()
            cache[s_id] = O.to_f64(datagen.keys(wl, s_id, q, w, seed), wl.dtype)
        K = cache[s_id]
        q_t = O.to_f64(q[t], wl.dtype)
        w_t = w[t].astype(np.float64)
        p = int(q_pos[t])
        t0 = time.perf_counter()
        if mode == "misa":
            O.misa_row(q_t, w_t, K, p, wl.block, wl.n_active_heads, wl.top_k)
        elif mode == "misa_dagger":
            O.misa_dagger_row(q_t, w_t, K, p, wl.block, wl.n_active_heads, wl.k_prime, wl.top_k)
        elif mode == "hisa":
            O.hisa_row(q_t, w_t, K, p, wl.block, wl.m_blocks, wl.top_k)
        elif mode == "misa_prefill":
            O.misa_row(q_t, w_t, K, p, 64, 8, wl.top_k)
        elif mode == "hisa_prefill":
            O.hisa_row(q_t, w_t, K, p, 128, 64, wl.top_k)
        elif mode == "misa_hisa":
            O.misa_hisa_row(q_t, w_t, K, p, wl.block, 8, wl.m_blocks, wl.top_k)
        elif mode == "certified":
            O.dosa_row(q_t, w_t, K, p, wl.top_k, 16)
        else:
            O.dense_row(q_t, w_t, K, p, wl.top_k)
        spent += time.perf_counter() - t0
        done_pairs += p + 1
        nq_done += 1
        if spent >= seconds:
            break
    return {"value": done_pairs / spent, "unit": "pair-scores/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{nq_done} of {wl.nq} query rows ({done_pairs} causal pairs), float64 NumPy, "
                      f"{spent:.1f} s of compute on {os.cpu_count()} visible host cores"}


def cpu_baseline_mla(wl, seed, seconds: float):
    """The attention oracle, as it stands, on whole queries of the same
    workload until about `seconds` of compute have run (row generation is
    not timed)."""
    import numpy as np

    import datagen
    from datagen import mla as M
    from oracle import attention as A
    q = M.queries(wl, seed)
    idx = M.index_lists(wl, seed)
    qs, _ = M.positions(wl)
    spent, done = 0.0, 0
    for t in range(wl.nq):
        rows = datagen.bf16_bits_to_f32(M.rows(wl, int(qs[t]), idx[t], seed)).astype(np.float64)
        q_t = datagen.bf16_bits_to_f32(q[t]).astype(np.float64)
        t0 = time.perf_counter()
        A.sparse_mla_row(q_t, rows, np.arange(wl.top_k), wl.d_v, wl.scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    return {"value": done * wl.top_k / spent, "unit": "attended (query, row) pairs/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {wl.nq} queries (all {wl.n_heads} heads, {wl.top_k} rows each), "
                      f"float64 NumPy, {spent:.1f} s of compute on {os.cpu_count()} visible host cores"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", default="read", choices=("read", "write"),
                    help="how cold-timed workloads evict the caches before each step")
    ap.add_argument("--l-max", type=int, default=None,
                    help="cache length of the hisa workload (default 1048576); at 131072 or "
                         "less the run also times the dense indexer on the same inputs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import datagen
    import sparse_attention_token_indexer_amd as dsa

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4,
                          "calibrate_copy_bytes_written": dst.numel() * 4}))
        return 0

    dsa.lib()
    name = args.workload
    extra = {}
    if name == "sparse_mla":
        from datagen import mla as M
        wl = M.WORKLOADS["sparse_mla_decode_L128K_H128"]
        nq, H, d, L, topk, eb = wl.nq, wl.n_heads, wl.d_qk, wl.l_max, wl.top_k, 2
        pairs = nq * topk                        # attended (query, listed row) pairs

        def bf16(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        mq = bf16(M.queries(wl, args.seed))
        idx_np = M.index_lists(wl, args.seed)
        qs_np, qp_np = M.positions(wl)
        # only the listed rows are ever read: they are generated and placed in
        # a zeroed cache of the full size
        kv = torch.zeros((wl.n_seq, L, d), dtype=torch.bfloat16, device=dev)
        for t in range(nq):
            kv[int(qs_np[t])][torch.from_numpy(idx_np[t].astype(np.int64)).to(dev)] = bf16(
                M.rows(wl, int(qs_np[t]), idx_np[t], args.seed))
        m_idx, m_qs, m_qp = (torch.from_numpy(x).to(dev) for x in (idx_np, qs_np, qp_np))
        m_out = torch.empty((nq, H, wl.d_v), dtype=torch.bfloat16, device=dev)
        nbytes = dsa.sparse_mla_workspace_size(nq, H, d, wl.d_v, topk)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

        def step():
            dsa.sparse_mla_attention(mq, kv, m_qp, m_idx, m_qs, softmax_scale=wl.scale,
                                     out=m_out, workspace=ws)
        kind = "mla"
        gathered = nq * topk * d * 2
        kernel_bytes = gathered + nq * H * d * 2 + nq * topk * 4 + nq * H * wl.d_v * 2
        call_bytes = kernel_bytes
        call_flops = 2 * nq * H * topk * (d + wl.d_v)
        bound_note = ("HBM: every listed latent row (1152 B) read once, plus the queries, the "
                      "lists and the outputs (the per-slice partial outputs are extra traffic)")
        extra["attention"] = {"d_qk": d, "d_v": wl.d_v, "softmax_scale": wl.scale}
    else:
        wl = datagen.WORKLOADS[WORKLOADS[name]]
        if name == "dense_shared_decode":
            # the dense decode workload's 64 queries on ONE shared 131072-key
            # cache (its last 64 positions): the shared-cache reading of a
            # decode batch, served by the query-grouped kernels
            wl = wl.replace(n_seq=1, layout="tail", name="dense_shared_decode_L128K_H64")
        if args.l_max is not None:
            if name != "hisa" or args.l_max < wl.m_blocks * wl.block:
                print("--l-max applies to the hisa workload, at least m * B = "
                      f"{wl.m_blocks * wl.block}", file=sys.stderr)
                return 2
            wl = wl.replace(l_max=args.l_max, name=f"hisa_decode_L{args.l_max // 1024}K_H32")
        inp = gen_inputs(wl, args.seed, dev)
        q, w, k, q_pos, q_seq = inp["q"], inp["w"], inp["k"], inp["q_pos"], inp["q_seq"]
        nq, H, d, L, topk = wl.nq, wl.n_heads, wl.head_dim, wl.l_max, wl.top_k
        eb = 2 if wl.dtype == datagen.BF16 else 4
        pos_np = inp["np"]["q_pos"]
        pairs = int((pos_np.astype(np.int64) + 1).sum())
        out_i = torch.empty((nq, topk), dtype=torch.int32, device=dev)
        out_s = torch.empty((nq, topk), dtype=torch.float32, device=dev)
        status = torch.zeros(nq, dtype=torch.int32, device=dev)       # HISA per-query status
        io_bytes = nq * H * d * eb + nq * H * 4 + nq * topk * 8       # q, w, outputs

    if name == "sparse_mla":
        pass
    elif name == "dense_shared_decode":
        nbytes = dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk, 0)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, out_idx=out_i,
                                   out_score=out_s, workspace=ws)
        kind = "prefill"
        kernel_bytes = None
        kernel_flops = pairs * H * d * 2
        call_bytes = nq * H * d * eb + L * d * eb + nq * H * 4 + nq * topk * 8
        call_flops = kernel_flops
        bound_note = ("MFMA: the head contraction of every causal (query, key) pair; the shared "
                      "cache is staged once per 8-query group")
    elif name == "certified":
        # the certified exact top-k (16 screened heads, bounds for the other 48,
        # survivors rescored with every head) on the dense decode inputs
        hs = 16
        nbytes = dsa.indexer_certified_topk_workspace_size(nq, H, d, wl.n_seq, L, hs, topk)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        surv = torch.zeros(nq, dtype=torch.int32, device=dev)

        def step():
            dsa.indexer_certified_topk(q, w, k, q_pos, q_seq, top_k=topk, n_screen_heads=hs,
                                       out_idx=out_i, out_score=out_s, out_survivors=surv,
                                       workspace=ws)
        step()
        torch.cuda.synchronize()
        n_surv = int(surv.sum())
        kind = "score_tokens"
        kernel_bytes = pairs * d * eb + nq * hs * d * eb + nq * hs * 4 + nq * topk * 8 + pairs * 4
        call_bytes = kernel_bytes + n_surv * (d * eb + 8) + nq * H * d * eb + nq * H * 4
        call_flops = pairs * hs * d * 2 + n_surv * H * d * 2
        bound_note = ("HBM: the screening pass reads every prefix key row once and writes its "
                      "upper bound")
        extra["certified"] = {"screened_heads": hs, "survivors": n_surv,
                              "survivor_frac": n_surv / pairs}
    elif name == "dense_prefill":
        nbytes = dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk, 0)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.indexer_score_topk(q, w, k, q_pos, None, top_k=topk, out_idx=out_i,
                                   out_score=out_s, workspace=ws)
        kind = "prefill"
        kernel_bytes = None
        kernel_flops = pairs * H * d * 2
        call_bytes = nq * H * d * eb + L * d * eb + nq * H * 4 + nq * topk * 8
        call_flops = kernel_flops
        bound_note = "MFMA: the head contraction of every causal (query, key) pair"
    elif name in ("dense_decode", "tiny"):
        nbytes = dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk,
                                                       0 if eb == 2 else 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, out_idx=out_i,
                                   out_score=out_s, workspace=ws)
        kind = "score_tokens"
        kernel_bytes = pairs * d * eb + io_bytes
        call_bytes, call_flops = kernel_bytes, pairs * H * d * 2
        bound_note = "HBM: every prefix key row is read once"
    elif name == "misa_prefill":
        h, B = 8, 64
        kp = dsa.indexer_mean_pool_keys(k, B)
        nbytes = dsa.misa_route_score_topk_workspace_size(nq, H, d, wl.n_seq, L, B, h, 0, topk, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.misa_route_score_topk(q, w, k, q_pos, None, block=B, n_active_heads=h,
                                      top_k=topk, k_pooled=kp, with_heads=False, out_idx=out_i,
                                      out_score=out_s, workspace=ws)
        kind = "prefill_routed"
        kernel_bytes = None
        kernel_flops = pairs * h * d * 2
        blocks = int(((pos_np.astype(np.int64) + B) // B).sum())      # causal pooled blocks
        call_bytes = nq * H * d * eb + L * d * eb + -(-L // B) * d * 2 + nq * H * 4 + nq * topk * 8
        call_flops = blocks * H * d * 2 + kernel_flops                  # router + routed pass
        bound_note = "MFMA: the routed heads' contraction of every causal (query, key) pair"
        extra["routing"] = {"h": h, "block": B}
    elif name in ("misa", "misa_dagger"):
        kp = dsa.indexer_mean_pool_keys(k, wl.block)
        kprime = wl.k_prime if name == "misa_dagger" else 0
        nbytes = dsa.misa_route_score_topk_workspace_size(nq, H, d, wl.n_seq, L, wl.block,
                                                          wl.n_active_heads, kprime, topk, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.misa_route_score_topk(q, w, k, q_pos, q_seq, block=wl.block,
                                      n_active_heads=wl.n_active_heads, top_k=topk, k_prime=kprime,
                                      k_pooled=kp, with_heads=False, out_idx=out_i,
                                      out_score=out_s, workspace=ws)
        kind = "score_tokens"
        h = wl.n_active_heads
        kernel_bytes = pairs * d * eb + nq * h * d * eb + nq * h * 4 + nq * (kprime or topk) * (4 if kprime else 8)
        M = -(-L // wl.block)
        call_bytes = pairs * d * eb + wl.n_seq * M * d * 2 + io_bytes   # keys + pooled + q, w, out
        call_flops = nq * H * M * d * 2 + pairs * h * d * 2               # router + routed pass
        if kprime:
            call_bytes += nq * kprime * (d * eb + 8)                       # gathered candidates
            call_flops += nq * kprime * H * d * 2                          # all-head rescoring
        bound_note = "HBM: the routed pass still reads every prefix key row"
    elif name == "hisa":
        kp = dsa.indexer_mean_pool_keys(k, wl.block)
        nbytes = dsa.hisa_block_filter_topk_workspace_size(nq, H, d, wl.n_seq, L, wl.block,
                                                           wl.m_blocks, topk, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.hisa_block_filter_topk(q, w, k, q_pos, q_seq, block=wl.block, m_blocks=wl.m_blocks,
                                       top_k=topk, k_pooled=kp, with_blocks=False, out_idx=out_i,
                                       out_score=out_s, out_status=status, workspace=ws)
        kind = "hisa"
        M = -(-L // wl.block)
        call_bytes = wl.n_seq * M * d * 2 + nq * wl.m_blocks * wl.block * d * eb + io_bytes
        call_flops = nq * M * H * d * 2 + nq * wl.m_blocks * wl.block * H * d * 2
        kernel_bytes = call_bytes          # one kernel: block pass, top-m, token pass, top-k
        bound_note = ("HBM: the pooled keys once and the keys of the m surviving blocks, in one "
                      "kernel (block pass, top-m, token pass, top-k)")
    elif name == "misa_hisa":
        h = 8
        kp = dsa.indexer_mean_pool_keys(k, wl.block)
        nbytes = dsa.misa_hisa_topk_workspace_size(nq, H, d, wl.n_seq, L, wl.block, h,
                                                   wl.m_blocks, topk, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.misa_hisa_topk(q, w, k, q_pos, q_seq, block=wl.block, n_active_heads=h,
                               m_blocks=wl.m_blocks, top_k=topk, k_pooled=kp, with_heads=False,
                               with_blocks=False, out_idx=out_i, out_score=out_s,
                               out_status=status, workspace=ws)
        kind = "hisa"
        M = -(-L // wl.block)
        pooled_bytes = wl.n_seq * M * d * 2
        gathered = nq * wl.m_blocks * wl.block * d * eb
        # the routed heads' q and w, the pooled keys, the kept blocks' keys, the outputs
        kernel_bytes = pooled_bytes + gathered + nq * h * (d * eb + 4) + nq * topk * 8
        call_bytes = pooled_bytes + gathered + io_bytes   # the router reads every head's q
        call_flops = (nq * M * H * d * 2 + nq * M * h * d * 2      # router + block pass
                      + nq * wl.m_blocks * wl.block * h * d * 2)  # token pass
        bound_note = ("HBM: the pooled keys once and the keys of the m surviving blocks, in one "
                      "kernel over the routed heads (block pass, top-m, token pass, top-k)")
        extra["routing"] = {"h": h, "block": wl.block, "m_blocks": wl.m_blocks}
    elif name == "hisa_prefill":
        B, m = 128, 64
        kp = dsa.indexer_mean_pool_keys(k, B)
        nbytes = dsa.hisa_block_filter_topk_workspace_size(nq, H, d, wl.n_seq, L, B, m, topk, 1)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

        def step():
            dsa.hisa_block_filter_topk(q, w, k, q_pos, None, block=B, m_blocks=m, top_k=topk,
                                       k_pooled=kp, with_blocks=False, out_idx=out_i,
                                       out_score=out_s, out_status=status, workspace=ws)
        kind = "hisa"
        kernel_bytes = None
        p1 = pos_np.astype(np.int64) + 1
        tokens = int(np.minimum(p1, m * B).sum())          # candidate tokens (at most m blocks)
        blocks = int(((p1 + B - 1) // B).sum())             # causal pooled blocks
        call_bytes = nq * H * d * eb + L * d * eb + -(-L // B) * d * 2 + nq * H * 4 + nq * topk * 8
        call_flops = blocks * H * d * 2 + tokens * H * d * 2
        kernel_flops = call_flops          # one kernel: block pass, top-m, token pass, top-k
        bound_note = ("MFMA: the head contraction over each row's pooled blocks and then its m "
                      "surviving blocks (keys re-gathered per row from L2 and the last-level cache)")
        extra["filter"] = {"block": B, "m_blocks": m}
    elif name == "pool":
        M = -(-L // wl.block)
        kp = torch.empty((wl.n_seq, M, d), dtype=torch.bfloat16, device=dev)

        def step():
            dsa.indexer_mean_pool_keys(k, wl.block, out=kp)
        kind = "pool"
        kernel_bytes = wl.n_seq * L * d * eb + wl.n_seq * M * d * 2
        call_bytes, call_flops = kernel_bytes, wl.n_seq * L * d
        bound_note = "HBM: reads the key cache once, writes the pooled keys"
    else:
        raise ValueError(name)

    # Workloads that touch less than the 256 MB last-level cache are timed cold:
    # before every step (outside its timing) a 512 MiB buffer is read through
    # (--flush read: the caches end up holding its clean lines) or overwritten
    # (--flush write: they end up holding dirty lines, whose write-back then
    # competes with the step's own reads).
    flush = None
    if name in ("hisa", "misa_hisa", "tiny", "sparse_mla"):
        flush_buf = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        if args.flush == "write":
            flush = lambda: flush_buf.zero_()
        else:
            flush = lambda: flush_buf.amax()

    def timed_region() -> float:
        """ms per step over args.steps steps (barrier + synchronize around)."""
        torch.cuda.synchronize()
        if flush is None:
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            t_start.record()
            for _ in range(args.steps):
                step()
            t_end.record()
            torch.cuda.synchronize()
            return t_start.elapsed_time(t_end) / args.steps
        total = 0.0
        for _ in range(args.steps):
            flush()
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            t_start.record()
            step()
            t_end.record()
            torch.cuda.synchronize()
            total += t_start.elapsed_time(t_end)
        return total / args.steps

    for _ in range(args.warmup):
        step()
    # pass 1: the call itself, nothing else on the stream
    ms_per_step = timed_region()
    # pass 2: the same steps with the library's per-launch HIP events on the
    # call's stream (they add a few microseconds per launch, so the call time
    # is taken from pass 1)
    dsa.kernel_timing(True)
    ms_per_step_events = timed_region()
    kt = dsa.kernel_timing_read(kind)
    per_kernel = {}
    for other in dsa.KERNEL_KINDS:
        if other == kind:
            continue
        r = dsa.kernel_timing_read(other)
        if r["launches"]:
            per_kernel[other] = round(r["total_ms"] / r["launches"] * 1e3, 2)
    dsa.kernel_timing(False)
    # pass 3: every call bracketed by its own events (median and minimum)
    per_call = []
    for _ in range(args.steps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1))
    per_call.sort()
    call_med_ms = per_call[len(per_call) // 2]
    if name == "hisa" and L <= 131072:
        # the dense indexer (all heads, every prefix key) on the same inputs,
        # timed the same way, for the HISA/dense latency ratio
        dws = torch.empty(dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk, 0),
                          dtype=torch.uint8, device=dev)
        d_i = torch.empty_like(out_i)
        d_s = torch.empty_like(out_s)

        def dense_step():
            dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, out_idx=d_i, out_score=d_s,
                                   workspace=dws)
        for _ in range(args.warmup):
            dense_step()
        dense_calls = []
        for _ in range(args.steps):
            if flush is not None:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            dense_step()
            e1.record()
            torch.cuda.synchronize()
            dense_calls.append(e0.elapsed_time(e1))
        dense_calls.sort()
        dense_med = dense_calls[len(dense_calls) // 2]
        extra["dense_same_inputs"] = {"call_median_us": dense_med * 1e3,
                                      "hisa_call_median_us": call_med_ms * 1e3,
                                      "dense_over_hisa": dense_med / call_med_ms}
    if name in ("hisa", "misa_hisa", "hisa_prefill"):
        extra["timed_out_queries"] = int(status.sum())       # of the last call (0: complete)
    if name == "certified":
        # the dense call on the same inputs (the same result), timed the same way
        dws = torch.empty(dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk, 0),
                          dtype=torch.uint8, device=dev)
        d_i = torch.empty_like(out_i)
        d_s = torch.empty_like(out_s)
        for _ in range(args.warmup):
            dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, out_idx=d_i, out_score=d_s,
                                   workspace=dws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, out_idx=d_i, out_score=d_s,
                                   workspace=dws)
        e1.record()
        torch.cuda.synchronize()
        same = bool(torch.equal(torch.sort(out_i, dim=1).values, torch.sort(d_i, dim=1).values))
        extra["dense_same_inputs"] = {"dense_us": e0.elapsed_time(e1) / args.steps * 1e3,
                                      "same_selection": same}
        del dws
    if name == "dense_shared_decode":
        # the same queries one short of the query-grouped path's 64: the
        # per-query decode kernels, which stream the shared cache per query
        dws = torch.empty(dsa.indexer_score_topk_workspace_size(nq - 1, H, d, 1, L, topk, 0),
                          dtype=torch.uint8, device=dev)
        qd, wd, pd = q[:-1].contiguous(), w[:-1].contiguous(), q_pos[:-1].contiguous()
        sd = q_seq[:-1].contiguous()
        for _ in range(args.warmup):
            dsa.indexer_score_topk(qd, wd, k, pd, sd, top_k=topk, with_scores=False, workspace=dws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dsa.indexer_score_topk(qd, wd, k, pd, sd, top_k=topk, with_scores=False, workspace=dws)
        e1.record()
        torch.cuda.synchronize()
        extra["decode_kernels_63_queries_us"] = e0.elapsed_time(e1) / args.steps * 1e3
        del dws
    if name in ("misa", "misa_dagger", "hisa", "misa_hisa") and L <= DENSE_IOU_MAX_L:
        # selection agreement of the last call's output with the dense indexer
        # on the same inputs (the IoU the MISA and HISA pages report)
        sel = out_i.clone()
        dws = torch.empty(dsa.indexer_score_topk_workspace_size(nq, H, d, wl.n_seq, L, topk, 0),
                          dtype=torch.uint8, device=dev)
        d_i, _ = dsa.indexer_score_topk(q, w, k, q_pos, q_seq, top_k=topk, with_scores=False,
                                        workspace=dws)
        iou = dsa.indexer_selection_iou(sel, d_i).cpu().numpy()
        extra["iou_vs_dense"] = {"mean": float(iou.mean()), "min": float(iou.min()),
                                 "queries": int(iou.size)}
        del dws
    k_avg_ms = kt["total_ms"] / max(kt["launches"], 1)
    per_kernel[kind] = round(k_avg_ms * 1e3, 2)
    traffic = stored_traffic(name)
    if kernel_bytes is None:       # compute-bound kernel
        achieved = kernel_flops / (k_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic, "kernel": kind,
                    "algorithmic_flops_per_launch": kernel_flops, "note": bound_note}
    else:
        achieved = kernel_bytes / (k_avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kind,
                    "algorithmic_bytes_per_launch": kernel_bytes, "note": bound_note}

    if name == "pool":
        metric, unit, value = "mean-pooled key-cache bytes/s", "GB/s", kernel_bytes / (ms_per_step * 1e-3) / 1e9
    elif name == "sparse_mla":
        metric = "sparse attention over the index lists: attended (query, row) pairs/s (1 MI355X)"
        unit = "pairs/s"
        value = pairs / (ms_per_step * 1e-3)
    else:
        metric = "indexer q·k pair-scores/sec + top-k latency at L=128K, H_I=64 (1 MI355X)"
        unit = "pair-scores/s"
        value = pairs / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline and name == "sparse_mla":
        cpu = cpu_baseline_mla(wl, args.seed, args.cpu_seconds)
    elif not args.no_cpu_baseline and name != "pool":
        cpu = cpu_baseline(wl, args.seed, args.cpu_seconds, name)

    line = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if eb == 2 else "f32",
        "data": "synthetic (seeded; planted-key recipe of the workload)",
        "config": {"workload": {"misa_dagger": "misa_dagger_decode_L128K_H64_h8_kp8192",
                                "pool": "mean_pool_L128K_B64",
                                "misa_prefill": "misa_prefill_L32K_H64_h8",
                                "hisa_prefill": "hisa_prefill_L32K_H64_B128_m64",
                                "misa_hisa": "misa_hisa_decode_L1M_H32_h8",
                                "certified": "certified_decode_L128K_H64_h16"}.get(name, wl.name),
                   "queries": nq, "l_max": L, "n_heads": H, "head_dim": d,
                   "top_k": topk, ("attended_pairs" if name == "sparse_mla" else "causal_pairs"): pairs,
                   "parallelism": "single GPU",
                   **({"block": wl.block} if getattr(wl, "block", 0) else {}),
                   **({"h": 8 if name == "misa_hisa" else wl.n_active_heads}
                      if name.startswith("misa") else {}),
                   **({"k_prime": wl.k_prime} if name == "misa_dagger" else {}),
                   **({"m_blocks": wl.m_blocks} if name in ("hisa", "misa_hisa") else {}),
                   **({"d_v": wl.d_v} if name == "sparse_mla" else {})},
        "topk_latency_us": ms_per_step * 1e3,
        "ms_per_step_with_kernel_events": ms_per_step_events,
        "call": {"latency_median_us": call_med_ms * 1e3, "latency_min_us": per_call[0] * 1e3,
                 "algorithmic_bytes": call_bytes, "algorithmic_flops": call_flops,
                 "gb_per_s": call_bytes / (ms_per_step * 1e-3) / 1e9,
                 "tflop_per_s": call_flops / (ms_per_step * 1e-3) / 1e12,
                 "hbm_frac": call_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "pair_scores_per_s": pairs / (ms_per_step * 1e-3),
                 "head_dots_per_s": call_flops / (2 * d) / (ms_per_step * 1e-3),
                 # the whole call's flops against the bf16 MFMA peak (next to the
                 # dominant kernel's fraction in roofline.frac)
                 "mfma_frac": call_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "cold_cache": (args.flush + " 512 MiB") if flush is not None else False,
        "kernel_avg_us": per_kernel,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "host": {"cpu_count": os.cpu_count(), "machine": platform.machine(),
                 "torch": torch.__version__},
        **extra,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
