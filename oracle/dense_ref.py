"""fp64 CPU oracle of the dense sibling operator (DenseLightningIndexerKLLossGrad).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

The metadata article ("DenseLightningIndexerKLLossGradMetadata", sections 导读,
功能定位, 约束说明 Mask and 总结) names the main operator, aclnnDenseLightningIndexerKLLossGrad,
and its interface limits: one key head, head dim 128, 1..128 query heads, BSND / TND
layouts, maskMode 0 (no mask) or 3 (rightDownCausal: the lower triangle whose corner
is the bottom-right vertex), and a key compression ratio cmpRatio in [1, 128] (with a
per-batch residual required when maskMode is 3 and cmpRatio is not 1).  Its formulas
are not on the pages.  Readings (also listed in the design notes):

D1. The dense operator is the sparse one ("aclnnSparseLightningIndexerKLLossGrad",
    formula section) with topk(t) replaced by every key the mask lets query t see:
    S = q_t K^T, I = W ReLU(S), y = Softmax(I) over the visible keys, dI = y - p,
    dW = dI ReLU(S)^T, dS = w (x) dI 1[S > 0], dq = dS K, dK += dS^T q.
D2. maskMode 0: query t of batch b sees all S2_b keys.  maskMode 3: it sees keys
    j <= t + (S2_b - S1_b) (rows and keys aligned at the bottom-right corner); a row
    that sees no key gives y = 0, dq = 0, dw = 0 and no dK term.
D3. p (attnSoftmaxL1Norm) and softmaxOut are dense over the key positions:
    [B, S1, N2, S2] | [T1, N2, S2max] (TND: S2max = the longest key sequence; positions
    at or past the row's batch key length, and masked ones, hold y = 0 and p is
    ignored there).
D4. Compression (cmpRatio > 1) is not defined on the pages; only cmpRatio = 1 is
    taken (the library rejects others as unsupported).
"""
from __future__ import annotations

import numpy as np

from .slikl_ref import BSND, TND, _row_table


def visible_keys(mask_mode: int, t: int, s1_b: int, s2_b: int) -> int:
    """Number of keys (a prefix 0 .. n-1) that query row t of a batch with s1_b rows
    and s2_b keys sees (reading D2)."""
    if mask_mode == 0:
        return s2_b
    if mask_mode == 3:
        return int(max(0, min(s2_b, t + (s2_b - s1_b) + 1)))
    raise ValueError("mask_mode must be 0 or 3")


def dense_grad_ref(q, k, w, p, *, mask_mode=3, layout_q=BSND, layout_k=BSND, cu_seqlens_q=None,
                   cu_seqlens_k=None, rows=None):
    """Dense operator in fp64, straight from the formulas over the visible keys.

    Shapes: q [B,S1,N1,D] | [T1,N1,D]; k [B,S2,N2,D] | [T2,N2,D]; w [B,S1,N1] |
    [T1,N1]; p [B,S1,N2,S2] | [T1,N2,S2max].  Returns dq, dk, dw, softmax_out (fp64,
    shaped like q, k, w and p)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    n1, d = q.shape[-2:]
    n2 = k.shape[-2]
    G = n1 // n2
    L = p.shape[-1]
    if layout_q == BSND:
        n_batch, s1 = q.shape[0], q.shape[1]
    else:
        n_batch, s1 = len(cu_seqlens_q) - 1, 0
    s2 = k.shape[1] if layout_k == BSND else 0
    qf, kf, wf, pf = q.reshape(-1, n1, d), k.reshape(-1, n2, d), w.reshape(-1, n1), p.reshape(-1, n2, L)
    dq, dk, dw = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(wf)
    y_out = np.zeros_like(pf)
    q_rows = _row_table(layout_q, n_batch, s1, cu_seqlens_q)
    k_rows = _row_table(layout_k, n_batch, s2, cu_seqlens_k)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(n_batch):
        q0, qlen = q_rows[b]
        k0, klen = k_rows[b]
        if klen > L:
            raise ValueError("a key sequence is longer than the dense axis of p")
        for t in range(qlen):
            r = q0 + t
            if wanted is not None and r not in wanted:
                continue
            n = visible_keys(mask_mode, t, qlen, klen)
            if n == 0:
                continue
            for g in range(n2):
                heads = slice(g * G, (g + 1) * G)
                K = kf[k0:k0 + n, g]                         # the visible keys
                S = qf[r, heads] @ K.T                       # [G, n]
                R = np.maximum(S, 0.0)
                I = wf[r, heads] @ R
                e = np.exp(I - I.max())
                y = e / e.sum()
                dI = y - pf[r, g, :n]
                dw[r, heads] = R @ dI
                dS = wf[r, heads][:, None] * dI[None, :] * (S > 0.0)
                dq[r, heads] = dS @ K
                dk[k0:k0 + n, g] += dS.T @ qf[r, heads]
                y_out[r, g, :n] = y
    return {"dq": dq.reshape(q.shape), "dk": dk.reshape(k.shape), "dw": dw.reshape(w.shape),
            "softmax_out": y_out.reshape(p.shape)}
