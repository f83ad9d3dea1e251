"""fp64 CPU oracle of the target distribution p (attnSoftmaxL1Norm).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

The operator page "aclnnSparseLightningIndexerKLLossGrad" says what p is in two
places: its function section (接口功能) says that the main attention branch
computes attnSoftmaxL1Norm beforehand and that the older fused operator
(SparseLightningIndexerGradKLLoss) recomputed the main attention inside its
kernel; its formula section (计算公式, the note after the softmax equation) says
that p equals what that older kernel formed from the main attention score by a
sum over heads and an L1 normalisation.  Readings where the page is silent
(each is also listed in the design notes):

P1. "Main attention score" is the main attention's softmax probability of head h
    for key j: P[h, j] = exp(z[h, j] - lse[h]) with z[h, j] = scale q_h . k_j
    (the usual scaled dot product; the scale is the caller's).
P2. lse[h] is the log-sum-exp of z[h, .] over the keys the main attention
    normalised over.  The caller may pass it (the main attention's forward keeps
    it); when it does not, the main attention is read as sparse over the same
    top-k keys, i.e. lse[h] = log sum over the valid slots of exp(z[h, s]).
P3. The sum over heads runs over the main-attention heads that share the key
    head of the index list: with N2 key heads and Nm query heads, key head g
    owns heads g Hm .. (g+1) Hm - 1, Hm = Nm / N2 (the group mapping of the
    indexer).  The key rows are those the indices name (batch-relative, -1 =
    no slot), exactly as for the indexer.
P4. The L1 normalisation runs over the valid slots of the unit:
    p[s] = a[s] / sum_{s' valid} a[s'] with a[s] = sum_h P[h, s];  p = 0 at -1
    slots, and a unit without a valid slot gives p = 0.  Duplicate indices are
    separate slots (each gets its own share).
With lse over exactly the valid slots, sum_s a[s] = Hm, so p is the head mean of
the per-head softmax; with lse over a larger key set the normalisation restricts
the heads' distributions to the top-k slots.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .slikl_ref import BSND, TND, _row_table


def attn_p_unit(qm_t, km_sel, valid, scale, lse_t=None):
    """One (query row, key head) unit in fp64.

    qm_t    [Hm, Dm]  main-attention queries of the unit's heads
    km_sel  [K, Dm]   key rows of the K top-k slots (rows of -1 slots ignored)
    valid   [K] bool  slot is a real index
    scale   float     softmax scale of the main attention
    lse_t   [Hm] or None: each head's log-sum-exp (reading P2)

    Returns p [K] (0 at -1 slots)."""
    K = km_sel.shape[0]
    p = np.zeros(K)
    v = np.flatnonzero(valid)
    if v.size == 0:
        return p
    z = scale * (qm_t @ km_sel[v].T)                  # [Hm, |V|]   reading P1
    if lse_t is None:                                 # reading P2: over the valid slots
        top = z.max(axis=1, keepdims=True)
        lse = top[:, 0] + np.log(np.exp(z - top).sum(axis=1))
    else:
        lse = np.asarray(lse_t, dtype=np.float64)
    P = np.exp(z - lse[:, None])                      # main-attention probabilities
    a = P.sum(axis=0)                                 # sum over heads      (P3)
    p[v] = a / a.sum()                                # L1 normalisation    (P4)
    return p


def attn_softmax_l1norm_ref(qm, km, sparse_indices, *, scale, lse=None, layout_q=BSND,
                            layout_k=BSND, cu_seqlens_q=None, cu_seqlens_k=None, rows=None):
    """Whole-tensor oracle of attnSoftmaxL1Norm, fp64.

    Shapes: qm [B,S1,Nm,Dm] | [T1,Nm,Dm]; km [B,S2,N2,Dm] | [T2,N2,Dm];
    sparse_indices [B,S1,N2,topk] | [T1,N2,topk]; lse (optional) [B,S1,Nm] | [T1,Nm].
    ``rows`` restricts the work to those flattened query rows (0 elsewhere).
    Returns p shaped like sparse_indices (float64)."""
    qm = np.asarray(qm, dtype=np.float64)
    km = np.asarray(km, dtype=np.float64)
    idx = np.asarray(sparse_indices, dtype=np.int64)
    nm, dm = qm.shape[-2:]
    n2 = km.shape[-2]
    if nm % n2:
        raise ValueError("the main-attention heads must be a multiple of the key heads")
    hm = nm // n2
    topk = idx.shape[-1]
    if layout_q == BSND:
        n_batch, s1 = qm.shape[0], qm.shape[1]
    else:
        n_batch, s1 = len(cu_seqlens_q) - 1, 0
    s2 = km.shape[1] if layout_k == BSND else 0
    qf = qm.reshape(-1, nm, dm)
    kf = km.reshape(-1, n2, dm)
    idxf = idx.reshape(-1, n2, topk)
    lf = None if lse is None else np.asarray(lse, dtype=np.float64).reshape(-1, nm)
    out = np.zeros(idxf.shape)
    q_rows = _row_table(layout_q, n_batch, s1, cu_seqlens_q)
    k_rows = _row_table(layout_k, n_batch, s2, cu_seqlens_k)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, klen = k_rows[b]
        for r in range(q0, q0 + qlen):
            if wanted is not None and r not in wanted:
                continue
            for g in range(n2):
                ids = idxf[r, g]
                valid = ids != -1
                if np.any(valid & ((ids < 0) | (ids >= klen))):
                    raise ValueError(f"row {r}: index outside the batch's key range")
                heads = slice(g * hm, (g + 1) * hm)
                km_sel = kf[np.where(valid, k0 + ids, k0), g] if klen else np.zeros((topk, dm))
                out[r, g] = attn_p_unit(qf[r, heads], km_sel, valid, scale,
                                        None if lf is None else lf[r, heads])
    return out.reshape(idx.shape)


def lse_over_slots_ref(qm, km, sparse_indices, *, scale, layout_q=BSND, layout_k=BSND,
                       cu_seqlens_q=None, cu_seqlens_k=None):
    """Each main-attention head's log-sum-exp of z over its unit's valid slots
    (reading P2), shaped [.., Nm]; heads of a unit without a valid slot get -inf."""
    qm = np.asarray(qm, dtype=np.float64)
    km = np.asarray(km, dtype=np.float64)
    idx = np.asarray(sparse_indices, dtype=np.int64)
    nm, dm = qm.shape[-2:]
    n2 = km.shape[-2]
    hm = nm // n2
    topk = idx.shape[-1]
    if layout_q == BSND:
        n_batch, s1 = qm.shape[0], qm.shape[1]
    else:
        n_batch, s1 = len(cu_seqlens_q) - 1, 0
    s2 = km.shape[1] if layout_k == BSND else 0
    qf, kf, idxf = qm.reshape(-1, nm, dm), km.reshape(-1, n2, dm), idx.reshape(-1, n2, topk)
    out = np.full((qf.shape[0], nm), -np.inf)
    q_rows = _row_table(layout_q, n_batch, s1, cu_seqlens_q)
    k_rows = _row_table(layout_k, n_batch, s2, cu_seqlens_k)
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, _ = k_rows[b]
        for r in range(q0, q0 + qlen):
            for g in range(n2):
                v = np.flatnonzero(idxf[r, g] != -1)
                if v.size == 0:
                    continue
                z = scale * (qf[r, g * hm:(g + 1) * hm] @ kf[k0 + idxf[r, g, v], g].T)
                top = z.max(axis=1, keepdims=True)
                out[r, g * hm:(g + 1) * hm] = top[:, 0] + np.log(np.exp(z - top).sum(axis=1))
    return out.reshape(qm.shape[:-1])
