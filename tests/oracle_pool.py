"""Full-size oracle results for the GPU parity tests, computed over row pieces in
parallel worker processes.

The oracle (``oracle.slikl_grad_ref`` and ``oracle.kl_per_unit_ref``) is called
unchanged on pieces of the problem: a piece is a run of query rows of ONE batch,
together with that batch's key sequence, passed as a one-sequence TND problem
(cuSeqLens [0, rows] and [0, keys]).  Batches never mix (indices are relative to
their batch), so the rows' dq, dw, softmaxOut and loss terms are exactly those
of the whole problem, and the whole dk is the sum over pieces of each piece's dk
placed at its batch's key base (an fp64 sum; only its rounding order differs from
one scatter-add over all rows).  That BSND and TND give the same results is one
of the oracle's pins.

Workers are started with the "spawn" method: they import numpy and the oracle
only, never torch or the GPU, and get their piece's arrays by pickling.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def _limit_threads():
    # one BLAS thread per worker: the pieces are the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:           # threadpoolctl missing: leave the default
        pass


def _piece(args):
    q, k, w, idx, p, want_kl = args
    from oracle import kl_per_unit_ref, slikl_grad_ref
    cu_q = np.array([0, q.shape[0]], dtype=np.int64)
    cu_k = np.array([0, k.shape[0]], dtype=np.int64)
    ref = slikl_grad_ref(q, k, w, idx, p, layout_q="TND", layout_k="TND",
                         cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, kink=True)
    out = {n: ref[n] for n in ("dq", "dk", "dw", "softmax_out", "dq_kink", "dk_kink", "logit_scale")}
    if want_kl:
        out["kl_loss"] = kl_per_unit_ref(q, k, w, idx, p, layout_q="TND", layout_k="TND",
                                         cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    return out


def workers() -> int:
    """Pool size: the CPUs this process may use, at most 16 (one GPU's host share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def batch_tables(x):
    """(first query row, rows, first key row, keys) of every batch, flattened."""
    n_batch = x.batch
    xq = x.q if hasattr(x, "q") else x.qm
    xk = x.k if hasattr(x, "k") else x.km
    if x.layout_q == "BSND":
        S1 = xq.shape[1]
        qt = [(b * S1, S1) for b in range(n_batch)]
    else:
        qt = [(int(x.cu_q[b]), int(x.cu_q[b + 1] - x.cu_q[b])) for b in range(n_batch)]
    if x.layout_k == "BSND":
        S2 = xk.shape[1]
        kt = [(b * S2, S2) for b in range(n_batch)]
    else:
        kt = [(int(x.cu_k[b]), int(x.cu_k[b + 1] - x.cu_k[b])) for b in range(n_batch)]
    return qt, kt


def oracle_full(x, *, batches=None, kl=True, n_workers=None, pieces_per_worker=4):
    """fp64 oracle outputs of the whole problem ``x`` (a workloads.Inputs), flattened:
    dq [T1,N1,D], dk [T2,N2,D], dw [T1,N1], softmax_out [T1,N2,topk], kl_loss
    [T1,N2] (with kl=True), and the oracle's kink allowances dq_kink / dk_kink and
    logit_scale.  ``batches`` restricts the work to those batches
    (other rows and keys stay 0).  Also returns ``rows``, the flat query rows
    computed."""
    n1, d = x.q.shape[-2:]
    n2 = x.k.shape[-2]
    topk = x.idx.shape[-1]
    qf = x.q.reshape(-1, n1, d)
    kf = x.k.reshape(-1, n2, d)
    wf = x.w.reshape(-1, n1)
    idxf = x.idx.reshape(-1, n2, topk)
    pf = x.p.reshape(-1, n2, topk)
    T1, T2 = qf.shape[0], kf.shape[0]
    qt, kt = batch_tables(x)
    todo = range(x.batch) if batches is None else batches
    nw = n_workers or workers()
    # cut the chosen batches into pieces of about equal valid-slot counts
    cost = (idxf >= 0).sum(axis=(1, 2)).astype(np.int64) + 64
    total = sum(int(cost[q0:q0 + n].sum()) for b in todo for q0, n in [qt[b]])
    target = max(1, total // (nw * pieces_per_worker))
    pieces = []
    for b in todo:
        q0, nq = qt[b]
        k0, nk = kt[b]
        start, acc = 0, 0
        for r in range(nq):
            acc += int(cost[q0 + r])
            if acc >= target or r == nq - 1:
                pieces.append((b, start, r + 1))
                start, acc = r + 1, 0
    out = dict(dq=np.zeros((T1, n1, d)), dk=np.zeros((T2, n2, d)), dw=np.zeros((T1, n1)),
               softmax_out=np.zeros((T1, n2, topk)), dq_kink=np.zeros((T1, n1, d)),
               dk_kink=np.zeros((T2, n2, d)), logit_scale=np.zeros((T1, n2)))
    if kl:
        out["kl_loss"] = np.zeros((T1, n2))
    args = []
    for b, r0, r1 in pieces:
        q0, _ = qt[b]
        k0, nk = kt[b]
        a, e = q0 + r0, q0 + r1
        args.append((qf[a:e], kf[k0:k0 + nk], wf[a:e], idxf[a:e], pf[a:e], kl))
    rows = []
    ctx = mp.get_context("spawn")
    step = max(1, len(pieces) // 10)
    with ctx.Pool(nw, initializer=_limit_threads) as pool:
        for i, ((b, r0, r1), res) in enumerate(zip(pieces, pool.imap(_piece, args))):
            if (i + 1) % step == 0 or i + 1 == len(pieces):
                print(f"[oracle] {i + 1}/{len(pieces)} pieces", flush=True)
            q0, _ = qt[b]
            k0, nk = kt[b]
            a, e = q0 + r0, q0 + r1
            for name in ("dq", "dw", "softmax_out", "dq_kink", "logit_scale") + (("kl_loss",) if kl else ()):
                out[name][a:e] = res[name]
            out["dk"][k0:k0 + nk] += res["dk"]
            out["dk_kink"][k0:k0 + nk] += res["dk_kink"]
            rows.append(np.arange(a, e))
    out["rows"] = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return out


def _attn_piece(args):
    qm, km, idx, scale, lse = args
    from oracle import attn_softmax_l1norm_ref
    cu_q = np.array([0, qm.shape[0]], dtype=np.int64)
    cu_k = np.array([0, km.shape[0]], dtype=np.int64)
    return attn_softmax_l1norm_ref(qm, km, idx, scale=scale, lse=lse, layout_q="TND", layout_k="TND",
                                   cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)


def attn_p_full(x, *, lse=None, n_workers=None, pieces_per_worker=4):
    """fp64 oracle of p for a whole workloads.AttnPInputs problem, flattened
    [T1, N2, topk], computed over row pieces (one batch each) in worker processes."""
    nm, dm = x.qm.shape[-2:]
    n2 = x.km.shape[-2]
    topk = x.idx.shape[-1]
    qf = x.qm.reshape(-1, nm, dm)
    kf = x.km.reshape(-1, n2, dm)
    idxf = x.idx.reshape(-1, n2, topk)
    lf = None if lse is None else np.asarray(lse).reshape(-1, nm)
    T1 = qf.shape[0]
    qt, kt = batch_tables(x)
    nw = n_workers or workers()
    cost = (idxf >= 0).sum(axis=(1, 2)).astype(np.int64) + 64
    target = max(1, int(cost.sum()) // (nw * pieces_per_worker))
    pieces = []
    for b in range(x.batch):
        q0, nq = qt[b]
        start, acc = 0, 0
        for r in range(nq):
            acc += int(cost[q0 + r])
            if acc >= target or r == nq - 1:
                pieces.append((b, start, r + 1))
                start, acc = r + 1, 0
    args = []
    for b, r0, r1 in pieces:
        q0, _ = qt[b]
        k0, nk = kt[b]
        a, e = q0 + r0, q0 + r1
        args.append((qf[a:e], kf[k0:k0 + nk], idxf[a:e], x.wl.scale, None if lf is None else lf[a:e]))
    out = np.zeros((T1, n2, topk))
    ctx = mp.get_context("spawn")
    step = max(1, len(pieces) // 10)
    with ctx.Pool(nw, initializer=_limit_threads) as pool:
        for i, ((b, r0, r1), res) in enumerate(zip(pieces, pool.imap(_attn_piece, args))):
            if (i + 1) % step == 0 or i + 1 == len(pieces):
                print(f"[oracle p] {i + 1}/{len(pieces)} pieces", flush=True)
            q0, _ = qt[b]
            out[q0 + r0:q0 + r1] = res
    return out
