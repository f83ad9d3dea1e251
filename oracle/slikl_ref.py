"""fp64 CPU oracle for the sparse lightning-indexer KL-loss backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

What it computes follows the operator page "aclnnSparseLightningIndexerKLLossGrad"
(CANN community edition API reference, ops-transformer):

* 计算公式 (formula section), equations S and I:  per query token t the
  top-k key rows K_topk(t) are gathered, S = q_t K_topk(t)^T per indexer head,
  I = W_t ReLU(S) (a weighted sum over heads);
* same section, softmax equation: y = Softmax(I), written to softmaxOut;
* same section, KL equations: L = sum_t KL(p_t || Softmax(I_t)) with p given
  by attnSoftmaxL1Norm;
* same section, gradient equations: dI = Softmax(I) - p, dW = dI ReLU(S)^T,
  dq = dS K_topk, dK_topk = dS^T q, scatter-added to the key rows named by
  sparseIndices; invalid (-1) top-k slots take no part;
* 约束说明 / 公共约束 (common constraints): BSND and TND layouts, TND needs
  cuSeqLens, valid indices lie inside the current batch's key range, padding
  is -1.

Readings of points the page leaves open (each is also listed in the design
notes):

1. dS is used but never defined on the page.  Reading: the chain rule through
   I = W ReLU(S), i.e. dS[h,s] = w[h] * dI[s] * 1[S[h,s] > 0] (ReLU'(0) = 0).
2. The softmax runs over the valid slots only; softmaxOut is 0 at -1 slots.
3. No 1/sqrt(d) scale and no temperature (the page's equations show none).
4. dI = y - p literally, whatever the sum of p over valid slots; p at -1
   slots is ignored.
5. Indices are batch-relative: key row = key base of the batch + index.
6. Duplicate indices in a row are independent slots (each takes part in the
   softmax and each scatter-adds into dK).
7. A row with no valid slot gives y = 0, dq = 0, dw = 0 and no dK term.
8. With N2 key heads, query head h belongs to key head h // (N1 / N2)
   (group size N1 / N2, as in the metadata article's groupSize_), and the
   top-k list, p and softmaxOut carry the N2 axis: [.., N2, topk].
9. Out-of-range indices (other than -1) violate the contract: the oracle
   raises.
10. seqUsedQ / seqUsedK (optional INT32 inputs of the constraints section; their
    meaning follows the sibling page's convention for TND, where a batch given 0
    takes no part): per batch of a TND side, the used length (clamped to the
    sequence's length).  Query rows past it take no part (all their outputs 0);
    the batch's key range is cut to it (indices past it are out of range).
11. The mask 1[S > 0] is a decision taken on a floating-point S.  An
    implementation that forms S in fp32 may take it the other way wherever S lies
    within fp32's rounding error of 0; both results are then correct.  With
    ``kink=True`` the oracle reports, per dq and dk element, the largest change
    such flips can make (see ``unit_backward``), for comparisons to allow.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

BSND = "BSND"
TND = "TND"
# fp32 unit roundoff
U32 = 2.0 ** -24


def gamma(n: int) -> float:
    """Worst-case relative error bound of an n-term fp32 sum of products, in any
    order: gamma_n = n u / (1 - n u) times the sum of the terms' magnitudes."""
    return n * U32 / (1.0 - n * U32)


def _used(rows, layout, used):
    """Cut each batch's length to its used length (TND side with a used array)."""
    if used is None or layout != TND:
        return rows
    used = np.asarray(used, dtype=np.int64)
    return [(s0, int(min(n, max(0, used[b])))) for b, (s0, n) in enumerate(rows)]


def _row_table(layout: str, n_batch: int, s: int, cu: Optional[np.ndarray]):
    """(start, length) of every batch along one side, in flattened rows."""
    if layout == BSND:
        return [(b * s, s) for b in range(n_batch)]
    if layout == TND:
        if cu is None:
            raise ValueError("TND layout needs cumulative sequence lengths")
        cu = np.asarray(cu, dtype=np.int64)
        if cu.shape != (n_batch + 1,) or cu[0] != 0 or np.any(np.diff(cu) < 0):
            raise ValueError("cumulative sequence lengths must start at 0 and not decrease")
        return [(int(cu[b]), int(cu[b + 1] - cu[b])) for b in range(n_batch)]
    raise ValueError(f"unknown layout {layout!r}")


def unit_backward(q_t, k_sel, valid, w_t, p_t, kink=False):
    """One (query token, key head) unit of the backward pass, in fp64.

    q_t    [G, D]   the token's queries for the G heads of this key head
    k_sel  [K, D]   gathered key rows for the K top-k slots (rows of -1 slots
                    are ignored; any finite values may sit there)
    valid  [K] bool slot is a real index (not -1)
    w_t    [G]      head weights
    p_t    [K]      target distribution (attnSoftmaxL1Norm row)

    Returns (y [K], dq_t [G, D], dw_t [G], dk_part [K, D]) where dk_part[s] is
    the row to scatter-add into the key named by slot s (zero for -1 slots).
    Follows the page's formula section equation by equation.

    With kink=True also returns (dq_kink [G, D], dk_kink [K, D], scale): the
    pairs (h, s) with |S| <= gamma_D sum_d |q_hd k_sd| are those whose mask an
    fp32 S may decide either way (reading 11); flipping the mask of pair (h, s)
    moves dq[h] by w_h dI_s K_s and the slot's dK part by w_h dI_s q_h, so
    dq_kink[h] = sum over its ambiguous pairs of |w_h dI_s| |K_s| and
    dk_kink[s] = sum over the slot's ambiguous pairs of |w_h dI_s| |q_h|
    (elementwise).  ``scale`` = max over valid slots of sum_h |w_h S_hs|, the
    magnitude of the terms that form I.
    """
    G, D = q_t.shape
    K = k_sel.shape[0]
    v = np.flatnonzero(valid)
    y = np.zeros(K)
    dq_t = np.zeros((G, D))
    dw_t = np.zeros(G)
    dk_part = np.zeros((K, D))
    if v.size == 0:                                       # reading 7
        if kink:
            return y, dq_t, dw_t, dk_part, np.zeros((G, D)), np.zeros((K, D)), 0.0
        return y, dq_t, dw_t, dk_part
    kv = k_sel[v]                                         # K_topk(t), valid slots only
    S = q_t @ kv.T                                        # eq. S: [G, |V|]
    R = np.maximum(S, 0.0)                                # ReLU(S)
    I = w_t @ R                                           # eq. I: [|V|]
    m = I.max()
    e = np.exp(I - m)
    yv = e / e.sum()                                      # y = Softmax(I) over valid slots
    dI = yv - p_t[v]                                      # dI = Softmax(I) - p
    dw_t = R @ dI                                         # dW = dI ReLU(S)^T
    dS = w_t[:, None] * dI[None, :] * (S > 0.0)           # reading 1
    dq_t = dS @ kv                                        # dq = dS K_topk
    dk_part[v] = dS.T @ q_t                               # dK_topk = dS^T q
    y[v] = yv
    if not kink:
        return y, dq_t, dw_t, dk_part
    amb = np.abs(S) <= gamma(D) * (np.abs(q_t) @ np.abs(kv).T)   # reading 11
    flip = np.abs(w_t)[:, None] * np.abs(dI)[None, :] * amb      # |w_h dI_s| on those pairs
    dq_kink = flip @ np.abs(kv)
    dk_kink = np.zeros((K, D))
    dk_kink[v] = flip.T @ np.abs(q_t)
    scale = float((np.abs(w_t) @ np.abs(S)).max())
    return y, dq_t, dw_t, dk_part, dq_kink, dk_kink, scale


def slikl_grad_ref(q, k, w, sparse_indices, p, *, layout_q=BSND, layout_k=BSND,
                   cu_seqlens_q=None, cu_seqlens_k=None, rows=None, seq_used_q=None,
                   seq_used_k=None, kink=False):
    """Whole-operator oracle.  Arrays are converted to fp64 on entry.

    Shapes: q [B,S1,N1,D] | [T1,N1,D]; k [B,S2,N2,D] | [T2,N2,D];
    w [B,S1,N1] | [T1,N1]; sparse_indices, p [B,S1,N2,topk] | [T1,N2,topk].

    ``rows`` (optional iterable of flattened query rows) restricts the work to
    those rows: the other rows of dq / dw / softmax_out stay 0 and dk holds
    only those rows' scatter-add terms.  ``seq_used_q`` / ``seq_used_k``: the
    used length of each batch of a TND side (reading 10).

    Returns a dict with fp64 ``dq``, ``dk``, ``dw``, ``softmax_out`` shaped
    like q, k, w and p.  With ``kink=True`` also ``dq_kink`` and ``dk_kink``
    (shaped like dq and dk: the largest change fp32 decisions of the mask at
    S near 0 can make to each element, reading 11) and ``logit_scale``
    ([..., N2] like p without its last axis: per unit, max over its valid slots
    of sum_h |w_h S_hs|).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    idx = np.asarray(sparse_indices, dtype=np.int64)

    if layout_q == BSND:
        n_batch, s1, n1, d = q.shape
    else:
        n_batch = len(cu_seqlens_q) - 1
        s1 = 0
        n1, d = q.shape[-2:]
    n2 = k.shape[-2]
    if n1 % n2:
        raise ValueError("N1 must be a multiple of N2")
    G = n1 // n2
    topk = idx.shape[-1]
    s2 = k.shape[1] if layout_k == BSND else 0
    if layout_k == BSND and k.shape[0] != n_batch:
        raise ValueError("q and k disagree on the batch size")
    if layout_k == TND and len(cu_seqlens_k) - 1 != n_batch:
        raise ValueError("cuSeqLensQ and cuSeqLensK disagree on the batch size")

    qf = q.reshape(-1, n1, d)
    kf = k.reshape(-1, n2, d)
    wf = w.reshape(-1, n1)
    idxf = idx.reshape(-1, n2, topk)
    pf = p.reshape(-1, n2, topk)
    T1, T2 = qf.shape[0], kf.shape[0]

    q_rows = _used(_row_table(layout_q, n_batch, s1, cu_seqlens_q), layout_q, seq_used_q)
    k_rows = _used(_row_table(layout_k, n_batch, s2, cu_seqlens_k), layout_k, seq_used_k)

    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dw = np.zeros_like(wf)
    y_out = np.zeros_like(pf)
    if kink:
        dq_k = np.zeros_like(qf)
        dk_k = np.zeros_like(kf)
        lscale = np.zeros(pf.shape[:2])

    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, klen = k_rows[b]
        for t in range(qlen):
            r = q0 + t
            if wanted is not None and r not in wanted:
                continue
            for g in range(n2):
                heads = slice(g * G, (g + 1) * G)
                ids = idxf[r, g]
                valid = ids != -1
                if np.any(valid & ((ids < 0) | (ids >= klen))):
                    raise ValueError(f"row {r}: index outside the batch's key range")
                krow = np.where(valid, k0 + ids, k0)      # key rows (dummy for -1)
                k_sel = kf[krow, g] if klen else np.zeros((topk, d))
                res = unit_backward(qf[r, heads], k_sel, valid, wf[r, heads], pf[r, g], kink=kink)
                y, dq_t, dw_t, dk_part = res[:4]
                y_out[r, g] = y
                dq[r, heads] = dq_t
                dw[r, heads] = dw_t
                vv = np.flatnonzero(valid)
                np.add.at(dk[:, g], krow[vv], dk_part[vv])   # scatter-add (duplicates add)
                if kink:
                    dq_k[r, heads] = res[4]
                    np.add.at(dk_k[:, g], krow[vv], res[5][vv])
                    lscale[r, g] = res[6]
    out = {
        "dq": dq.reshape(q.shape),
        "dk": dk.reshape(k.shape),
        "dw": dw.reshape(w.shape),
        "softmax_out": y_out.reshape(p.shape),
        "T1": T1,
        "T2": T2,
    }
    if kink:
        out["dq_kink"] = dq_k.reshape(q.shape)
        out["dk_kink"] = dk_k.reshape(k.shape)
        out["logit_scale"] = lscale.reshape(p.shape[:-1])
    return out


def kl_loss_ref(q, k, w, sparse_indices, p, *, layout_q=BSND, layout_k=BSND,
                cu_seqlens_q=None, cu_seqlens_k=None):
    """L = sum over tokens and key heads of KL(p || Softmax(I)) over valid slots.

    Formula section, KL equations (0 log 0 = 0).  Used by the finite-difference
    pins of the gradients.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    idx = np.asarray(sparse_indices, dtype=np.int64)
    if layout_q == BSND:
        n_batch, s1, n1, d = q.shape
    else:
        n_batch, s1 = len(cu_seqlens_q) - 1, 0
        n1, d = q.shape[-2:]
    n2 = k.shape[-2]
    G = n1 // n2
    topk = idx.shape[-1]
    s2 = k.shape[1] if layout_k == BSND else 0
    qf, kf = q.reshape(-1, n1, d), k.reshape(-1, n2, d)
    wf, idxf, pf = w.reshape(-1, n1), idx.reshape(-1, n2, topk), p.reshape(-1, n2, topk)
    q_rows = _row_table(layout_q, n_batch, s1, cu_seqlens_q)
    k_rows = _row_table(layout_k, n_batch, s2, cu_seqlens_k)
    total = 0.0
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, _ = k_rows[b]
        for t in range(qlen):
            r = q0 + t
            for g in range(n2):
                ids = idxf[r, g]
                v = np.flatnonzero(ids != -1)
                if v.size == 0:
                    continue
                kv = kf[k0 + ids[v], g]
                I = wf[r, g * G:(g + 1) * G] @ np.maximum(qf[r, g * G:(g + 1) * G] @ kv.T, 0.0)
                logy = I - I.max() - np.log(np.exp(I - I.max()).sum())
                pv = pf[r, g, v]
                nz = pv > 0
                total += float(np.sum(pv[nz] * (np.log(pv[nz]) - logy[nz])))
    return total


def kl_per_unit_ref(q, k, w, sparse_indices, p, *, layout_q=BSND, layout_k=BSND,
                    cu_seqlens_q=None, cu_seqlens_k=None, rows=None, seq_used_q=None,
                    seq_used_k=None):
    """KL(p_u || Softmax(I_u)) of every (query row, key head) unit u, fp64, shaped
    [T1, N2]: the terms of the formula section's loss L before its sum over tokens.
    ``rows`` (optional flattened query rows) restricts the work to them (0 elsewhere).

    Per unit: over its valid slots, log y_s = I_s - logsumexp(I); the unit's value is
    sum of p_s (log p_s - log y_s) over the valid slots with p_s > 0 (0 log 0 = 0;
    duplicate slots count separately).  A unit with no valid slot gives 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    idx = np.asarray(sparse_indices, dtype=np.int64)
    n1, d = q.shape[-2:]
    n2 = k.shape[-2]
    G = n1 // n2
    topk = idx.shape[-1]
    if layout_q == BSND:
        n_batch, s1 = q.shape[0], q.shape[1]
    else:
        n_batch, s1 = len(cu_seqlens_q) - 1, 0
    s2 = k.shape[1] if layout_k == BSND else 0
    qf, kf = q.reshape(-1, n1, d), k.reshape(-1, n2, d)
    wf, idxf, pf = w.reshape(-1, n1), idx.reshape(-1, n2, topk), p.reshape(-1, n2, topk)
    out = np.zeros((qf.shape[0], n2))
    q_rows = _used(_row_table(layout_q, n_batch, s1, cu_seqlens_q), layout_q, seq_used_q)
    k_rows = _used(_row_table(layout_k, n_batch, s2, cu_seqlens_k), layout_k, seq_used_k)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, _ = k_rows[b]
        for r in range(q0, q0 + qlen):
            if wanted is not None and r not in wanted:
                continue
            for g in range(n2):
                heads = slice(g * G, (g + 1) * G)
                v = np.flatnonzero(idxf[r, g] != -1)
                if v.size == 0:
                    continue
                S = qf[r, heads] @ kf[k0 + idxf[r, g, v], g].T          # eq. S
                I = wf[r, heads] @ np.maximum(S, 0.0)                    # eq. I
                top = I.max()
                logy = I - (top + np.log(np.sum(np.exp(I - top))))       # log Softmax(I)
                pv = pf[r, g, v]
                pos = pv > 0
                out[r, g] = np.sum(pv[pos] * (np.log(pv[pos]) - logy[pos]))
    return out
