"""Driver of the host-side bounds audit (run by tests/test_audit_cpu.py in a
process of its own, with the address sanitizer's runtime preloaded).

It loads libdsa_audit.so - the library's C-ABI layer compiled for the host,
linked with tests/audit/kernel_model.cpp in place of the kernels - and calls
every entry point with fake device addresses: each input, output and the
workspace (at the size the library asks for) is a registered buffer of its
exact byte size, never dereferenced on the host.  q_seq / q_pos contents are
registered too, since the kernels read them.  Every modelled kernel access must
fall inside one registered buffer.

Usage: python drive.py LIB  -> prints one JSON line {"cases": n, "violations": [...],
"launches": {...}}; exit status 1 when any case had a violation.
"""
from __future__ import annotations

import ctypes
import importlib.util
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
_spec = importlib.util.spec_from_file_location(
    "_dsa_abi", os.path.join(ROOT, "sparse_attention_token_indexer_amd", "_abi.py"))
_abi = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_abi)

BF16, F32 = 0, 1


class Audit:
    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        for name, (args, res) in _abi._SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        L.audit_region.argtypes = [ctypes.c_uint64, ctypes.c_size_t, ctypes.c_char_p]
        L.audit_ints.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64]
        L.audit_report.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        L.audit_report.restype = ctypes.c_int
        L.audit_launches.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        self.L = L
        self.viol = []
        self.launches = {}
        self.cases = 0

    # -- fake device buffers
    def reset(self):
        self.L.audit_reset()
        self.next = 1 << 44

    def buf(self, nbytes: int, name: str) -> int:
        base = self.next
        self.next += ((max(int(nbytes), 1) + (1 << 30)) >> 30 << 30) + (1 << 30)
        self.L.audit_region(base, int(nbytes), name.encode())
        return base

    def ints(self, vals, name: str) -> int:
        a = np.ascontiguousarray(np.asarray(vals, dtype=np.int32))
        p = self.buf(a.nbytes, name)
        self.L.audit_ints(p, a.ctypes.data, a.size)
        return p

    def finish(self, tag: str, st: int, expect_ok: bool = True):
        self.cases += 1
        buf = ctypes.create_string_buffer(1 << 16)
        n = self.L.audit_report(buf, len(buf))
        if n:
            self.viol.append(f"[{tag}] " + buf.value.decode())
        if expect_ok and st != 0:
            self.viol.append(f"[{tag}] status {st}: {self.L.dsa_last_error().decode()}")
        lb = ctypes.create_string_buffer(4096)
        self.L.audit_launches(lb, len(lb))
        for item in lb.value.decode().split(";"):
            if item:
                k, v = item.split("=")
                self.launches[k] = self.launches.get(k, 0) + int(v)
        return st

    # -- common inputs
    def inputs(self, nq, H, d, n_seq, L, dtype, q_seq, q_pos):
        eb = 2 if dtype == BF16 else 4
        return dict(q=self.buf(nq * H * d * eb, "q"), w=self.buf(nq * H * 4, "w"),
                    k=self.buf(n_seq * L * d * eb, "k"),
                    q_seq=None if q_seq is None else self.ints(q_seq, "q_seq"),
                    q_pos=self.ints(q_pos, "q_pos"))


def positions(layout, nq, n_seq, L, rng=None, invalid=0.0):
    t = np.arange(nq)
    if layout == "decode":
        seq, pos = t % n_seq, np.full(nq, L - 1)
    elif layout == "tail":
        seq, pos = np.zeros(nq, int), np.maximum(L - nq + t, 0)
    elif layout == "prefill":
        seq, pos = np.zeros(nq, int), np.minimum(t, L - 1)
    else:   # random
        seq, pos = rng.integers(0, n_seq, nq), rng.integers(0, L, nq)
    if invalid and rng is not None:
        bad = rng.random(nq) < invalid
        kind = rng.integers(0, 4, nq)
        pos = np.where(bad & (kind == 0), -1, pos)
        pos = np.where(bad & (kind == 1), L, pos)
        seq = np.where(bad & (kind == 2), n_seq, seq)
        seq = np.where(bad & (kind == 3), -1, seq)
    return seq, pos


def run_dense(A, tag, nq, H, d, n_seq, L, k, dtype=BF16, layout="decode", rng=None, invalid=0.0,
              with_seq=True, scores=True):
    A.reset()
    seq, pos = positions(layout, nq, n_seq, L, rng, invalid)
    x = A.inputs(nq, H, d, n_seq, L, dtype, seq if with_seq else None, pos)
    ws = A.L.indexer_score_topk_workspace_size(nq, H, d, n_seq, L, k, dtype)
    st = A.L.indexer_score_topk(x["q"], x["w"], x["k"], dtype, x["q_seq"], x["q_pos"], nq, H, d,
                                n_seq, L, k, A.buf(nq * k * 4, "out_idx"),
                                A.buf(nq * k * 4, "out_score") if scores else None,
                                A.buf(ws, "workspace"), ws, None)
    return A.finish(tag, st)


def run_cert(A, tag, nq, H, d, n_seq, L, h, k, layout="decode", rng=None, invalid=0.0,
             surv=True):
    A.reset()
    seq, pos = positions(layout, nq, n_seq, L, rng, invalid)
    x = A.inputs(nq, H, d, n_seq, L, BF16, seq, pos)
    ws = A.L.indexer_certified_topk_workspace_size(nq, H, d, n_seq, L, h, k)
    st = A.L.indexer_certified_topk(x["q"], x["w"], x["k"], BF16, x["q_seq"], x["q_pos"], nq, H, d,
                                    n_seq, L, h, k, A.buf(nq * k * 4, "out_idx"),
                                    A.buf(nq * k * 4, "out_score"),
                                    A.buf(nq * 4, "out_survivors") if surv else None,
                                    A.buf(ws, "workspace"), ws, None)
    return A.finish(tag, st)


def run_misa(A, tag, nq, H, d, n_seq, L, B, h, kp, k, pooled=True, layout="decode", rng=None,
             invalid=0.0, outs=True):
    A.reset()
    seq, pos = positions(layout, nq, n_seq, L, rng, invalid)
    x = A.inputs(nq, H, d, n_seq, L, BF16, seq, pos)
    M = -(-L // B)
    ws = A.L.misa_route_score_topk_workspace_size(nq, H, d, n_seq, L, B, h, kp, k, int(pooled))
    st = A.L.misa_route_score_topk(
        x["q"], x["w"], x["k"], A.buf(n_seq * M * d * 2, "k_pooled") if pooled else None, BF16,
        x["q_seq"], x["q_pos"], nq, H, d, n_seq, L, B, h, kp, k, A.buf(nq * k * 4, "out_idx"),
        A.buf(nq * k * 4, "out_score"), A.buf(nq * h * 4, "out_heads") if outs else None,
        A.buf(nq * H * 4, "out_importance") if outs else None,
        A.buf(nq * kp * 4, "out_cand") if (outs and kp) else None, A.buf(ws, "workspace"), ws,
        None)
    return A.finish(tag, st)


def run_hisa(A, tag, nq, H, d, n_seq, L, B, m, k, pooled=True, layout="decode", rng=None,
             invalid=0.0, outs=True, h=0):
    A.reset()
    seq, pos = positions(layout, nq, n_seq, L, rng, invalid)
    x = A.inputs(nq, H, d, n_seq, L, BF16, seq, pos)
    M = -(-L // B)
    kpool = A.buf(n_seq * M * d * 2, "k_pooled") if pooled else None
    blocks = A.buf(nq * m * 4, "out_blocks") if outs else None
    bsc = A.buf(nq * m * 4, "out_block_score") if outs else None
    status = A.buf(nq * 4, "out_status") if outs else None
    if h:
        ws = A.L.misa_hisa_topk_workspace_size(nq, H, d, n_seq, L, B, h, m, k, int(pooled))
        st = A.L.misa_hisa_topk(x["q"], x["w"], x["k"], kpool, BF16, x["q_seq"], x["q_pos"], nq, H,
                                d, n_seq, L, B, h, m, k, A.buf(nq * k * 4, "out_idx"),
                                A.buf(nq * k * 4, "out_score"),
                                A.buf(nq * h * 4, "out_heads") if outs else None,
                                A.buf(nq * H * 4, "out_importance") if outs else None, blocks, bsc,
                                status, A.buf(ws, "workspace"), ws, None)
    else:
        ws = A.L.hisa_block_filter_topk_workspace_size(nq, H, d, n_seq, L, B, m, k, int(pooled))
        st = A.L.hisa_block_filter_topk(x["q"], x["w"], x["k"], kpool, BF16, x["q_seq"], x["q_pos"],
                                        nq, H, d, n_seq, L, B, m, k, A.buf(nq * k * 4, "out_idx"),
                                        A.buf(nq * k * 4, "out_score"), blocks, bsc, status,
                                        A.buf(ws, "workspace"), ws, None)
    fused_limits = m > 1024 or m * B > 8192 or -(-L // B) > 64 * 2048 or nq > 65535
    return A.finish(tag, st, expect_ok=not (h and fused_limits))


def run_pool(A, tag, n_seq, L, d, B):
    A.reset()
    st = A.L.indexer_mean_pool_keys(A.buf(n_seq * L * d * 2, "k"), BF16, n_seq, L, d, B,
                                    A.buf(n_seq * -(-L // B) * d * 2, "k_pooled"), None)
    return A.finish(tag, st)


def run_iou(A, tag, nq, k):
    A.reset()
    st = A.L.indexer_selection_iou(A.buf(nq * k * 4, "a"), A.buf(nq * k * 4, "b"), nq, k,
                                   A.buf(nq * 4, "out_iou"), None)
    return A.finish(tag, st)


def run_mla(A, tag, nq, H, n_seq, L, k, layout="decode", rng=None, invalid=0.0):
    A.reset()
    seq, pos = positions(layout, nq, n_seq, L, rng, invalid)
    ws = A.L.sparse_mla_workspace_size(nq, H, 576, 512, k)
    st = A.L.sparse_mla_attention(A.buf(nq * H * 576 * 2, "q"), A.buf(n_seq * L * 576 * 2, "kv"),
                                  BF16, A.ints(seq, "q_seq"), A.ints(pos, "q_pos"),
                                  A.buf(nq * k * 4, "idx"), nq, H, 576, 512, n_seq, L, k, 0.07,
                                  A.buf(nq * H * 512 * 2, "out"), A.buf(ws, "workspace"), ws, None)
    return A.finish(tag, st)


def workloads(A):
    """Every workload at its full size, and the calls of the full-size tests."""
    # the full-size HISA test: HISA, the dense 32-head indexer and the IoU at
    # 32 queries x 1048576 keys (B 128, m 64, k 2048)
    L5 = 1 << 20
    for pooled in (True, False):
        run_pool(A, "pool C5", 32, L5, 128, 128)
        run_hisa(A, f"hisa C5 pooled={pooled}", 32, 32, 128, 32, L5, 128, 64, 2048, pooled)
        run_hisa(A, f"misa-hisa C5 pooled={pooled}", 32, 32, 128, 32, L5, 128, 64, 2048, pooled,
                 h=8)
    run_dense(A, "dense C5 shape (32 x 1M, 32 heads)", 32, 32, 128, 32, L5, 2048)
    run_dense(A, "dense C5 shape, no scores", 32, 32, 128, 32, L5, 2048, scores=False)
    run_iou(A, "iou 32 x 2048", 32, 2048)
    # dense decode, MISA / MISA dagger, tiny, prefill shapes, sparse attention
    run_dense(A, "dense C2", 64, 64, 128, 64, 131072, 2048)
    run_cert(A, "certified C2, 16 screened heads", 64, 64, 128, 64, 131072, 16, 2048)
    run_cert(A, "certified short rows (short passes)", 64, 64, 128, 64, 9000, 8, 2048)
    run_pool(A, "pool C4", 64, 131072, 128, 64)
    run_misa(A, "misa C4", 64, 64, 128, 64, 131072, 64, 8, 0, 2048)
    run_misa(A, "misa dagger C4", 64, 64, 128, 64, 131072, 64, 8, 8192, 2048)
    run_iou(A, "iou 64 x 2048", 64, 2048)
    run_dense(A, "tiny C1", 16, 8, 64, 1, 4096, 64, dtype=F32, layout="tail")
    run_dense(A, "dense prefill C3", 32768, 64, 128, 1, 32768, 2048, layout="prefill",
              with_seq=False)
    run_misa(A, "misa prefill C3", 32768, 64, 128, 1, 32768, 64, 8, 0, 2048, pooled=False,
             layout="prefill")
    run_hisa(A, "hisa prefill C3", 32768, 64, 128, 1, 32768, 128, 64, 2048, layout="prefill")
    # prefill-shaped calls whose rows outgrow 16-bit counts or whose row groups
    # are too few to fill the chip: keys split over workgroups, 11-bit bins
    run_dense(A, "dense shared-cache decode 64 x 131072", 64, 64, 128, 1, 131072, 2048,
              layout="tail")
    run_misa(A, "misa shared-cache decode 64 x 131072", 64, 64, 128, 1, 131072, 64, 8, 0, 2048,
             pooled=False, layout="tail")
    run_dense(A, "dense prefill chunk 96 x 100000", 96, 64, 128, 1, 100000, 2048,
              layout="prefill", with_seq=False)
    run_dense(A, "dense long rows 2048 x 70000", 2048, 64, 128, 1, 70000, 2048, layout="tail")
    run_mla(A, "sparse attention 64 x 128 heads x 2048", 64, 128, 64, 131072, 2048)
    run_mla(A, "sparse attention 256 queries (unsplit)", 256, 128, 256, 4096, 2048)


def sweep(A, n, seed):
    """Random shapes, positions (some invalid) and options for every entry point."""
    rng = np.random.default_rng(seed)
    for i in range(n):
        nq = int(rng.choice([1, 3, 8, 33, 64, 65, 200, 700]))
        L = int(rng.choice([1, 7, 100, 2047, 4096, 9000, 65535, 65536, 70000, 200000]))
        n_seq = int(rng.integers(1, 5)) if rng.random() < 0.5 else nq
        H = int(rng.choice([1, 5, 8, 16, 17, 32, 33, 48, 64]))
        d = int(rng.choice([64, 128]))
        k = int(rng.choice([1, 16, 64, 300, 2048, 5000]))
        layout = str(rng.choice(["decode", "tail", "prefill", "random"]))
        if layout == "decode":
            n_seq = nq
        if layout in ("tail", "prefill"):
            n_seq = 1
        inv = float(rng.choice([0.0, 0.2]))
        tag = f"sweep {i}: nq={nq} L={L} n_seq={n_seq} H={H} d={d} k={k} {layout} invalid={inv}"
        run_dense(A, tag + " dense", nq, H, d, n_seq, L, k, layout=layout, rng=rng, invalid=inv,
                  with_seq=layout != "prefill" or rng.random() < 0.5)
        if d == 64 and L <= 70000 and nq <= 64:
            run_dense(A, tag + " dense f32", nq, H, d, n_seq, L, k, dtype=F32, layout=layout,
                      rng=rng, invalid=inv)
        B = int(rng.choice([1, 16, 64, 128, 300]))
        h = int(rng.integers(1, H + 1))
        kp = int(rng.choice([0, 0, k, 2 * k, 9000])) if k <= 5000 else 0
        run_misa(A, tag + f" misa B={B} h={h} k'={kp}", nq, H, d, n_seq, L, B, h, kp, k,
                 pooled=bool(rng.random() < 0.5), layout=layout, rng=rng, invalid=inv,
                 outs=bool(rng.random() < 0.7))
        m = int(rng.choice([1, 4, 16, 64, 200, 1100]))
        run_hisa(A, tag + f" hisa B={B} m={m}", nq, H, d, n_seq, L, B, m, k,
                 pooled=bool(rng.random() < 0.5), layout=layout, rng=rng, invalid=inv,
                 outs=bool(rng.random() < 0.7))
        run_hisa(A, tag + f" misa-hisa B={B} h={h} m={m}", nq, H, d, n_seq, L, B, m, k,
                 pooled=bool(rng.random() < 0.5), layout=layout, rng=rng, invalid=inv, h=h)
        if H % 32 == 0 or rng.random() < 0.3:
            Hm = int(rng.choice([32, 64, 96, 128]))
            km = int(rng.choice([1, 31, 33, 2048, 4096, 32768]))
            run_mla(A, tag + f" mla H={Hm} k={km}", nq, Hm, n_seq, L, km, layout=layout, rng=rng,
                    invalid=inv)
        run_iou(A, tag + " iou", nq, min(k, 8192))
        if H <= 64:
            hc = int(rng.integers(1, min(H, 16) + 1))
            run_cert(A, tag + f" certified h={hc}", nq, H, d, n_seq, L, hc, k, layout=layout,
                     rng=rng, invalid=inv, surv=bool(rng.random() < 0.7))


def planted(A):
    """The audit must see a buffer that is too small: the same calls with one
    buffer cut short by one element each time.  Returns the cases that went
    undetected."""
    missed = []
    real_buf = A.buf

    def run(tag, victim, cut, fn):
        def buf(nbytes, name):
            return real_buf(nbytes - cut if name == victim else nbytes, name)
        A.buf = buf
        n0 = len(A.viol)
        fn()
        A.buf = real_buf
        if len(A.viol) == n0:
            missed.append(f"{tag}: {victim} cut by {cut} bytes not detected")
        del A.viol[n0:]

    L5 = 1 << 20
    hisa = lambda: run_hisa(A, "p", 32, 32, 128, 32, L5, 128, 64, 2048)
    dense = lambda: run_dense(A, "p", 32, 32, 128, 32, L5, 2048)
    for victim in ("k", "k_pooled", "out_idx", "out_score", "out_blocks", "out_status", "q", "w"):
        run("hisa C5", victim, 4, hisa)
    for victim in ("k", "out_idx", "out_score", "workspace", "q", "q_pos"):
        run("dense C5 shape", victim, 4, dense)
    run("iou", "b", 4, lambda: run_iou(A, "p", 32, 2048))
    run("misa dagger", "out_cand", 4,
        lambda: run_misa(A, "p", 64, 64, 128, 64, 131072, 64, 8, 8192, 2048))
    run("prefill", "workspace", 16,       # (the last row's metadata word 3 is unused)
        lambda: run_dense(A, "p", 32768, 64, 128, 1, 32768, 2048, layout="prefill",
                          with_seq=False))
    cert = lambda: run_cert(A, "p", 64, 64, 128, 64, 131072, 16, 2048)
    for victim in ("k", "q", "w", "out_idx", "out_score", "out_survivors", "workspace"):
        run("certified C2", victim, 4, cert)
    run("sparse attention", "kv", 2, lambda: run_mla(A, "p", 64, 128, 64, 131072, 2048))
    run("sparse attention", "workspace", 4, lambda: run_mla(A, "p", 64, 128, 64, 131072, 2048))
    return missed


def main():
    A = Audit(sys.argv[1])
    n_sweep = int(sys.argv[2]) if len(sys.argv) > 2 else 60
    workloads(A)
    sweep(A, n_sweep, 7)
    missed = planted(A)
    print(json.dumps({"cases": A.cases, "violations": A.viol, "launches": A.launches,
                      "planted_missed": missed}))
    return 1 if (A.viol or missed) else 0


if __name__ == "__main__":
    sys.exit(main())
