"""Reference for the load-balancing metadata (integer work, must match bit for bit).

TEST INFRASTRUCTURE ONLY (see slikl_ref.py).  It does not import the product.

Prior art: the article "在 CANN ops-transformer 中理解
DenseLightningIndexerKLLossGradMetadata：用于负载均衡的分核 metadata 生成器"
describes, in its 功能定位 section, a pre-pass that merges the B and S1 axes,
sums the per-batch query lengths into totalNum (CalcSplitInfo), and splits the
rows over the cores with formerCoreProcessNum = CeilDiv(totalNum, cores),
remainCoreProcessNum = formerCoreProcessNum - 1, a count of cores that take the
smaller share, and a used-core count (GenMetadata); its Metadata 输出布局
section lists those fields first in a fixed INT32 array.

The article gives only the names of the remainder fields.  Reading: with P
parts and U >= 1 units, former = ceil(U / P), remain = former - 1,
remain_num = P * former - U, former_num = P - remain_num; the first former_num
parts take `former` units each and the rest take `remain` units; used parts are
those with at least one unit.

This library's layout is its own (the sparse operator's metadata format is not
on the operator page).  A unit is one (query row, key head) pair,
u = row * N2 + g.  Besides the article's even row split ("rows" mode) it has a
"weighted" mode: unit cost c_u = (valid slots of u) + overhead, and part i
starts at the first unit u whose exclusive cost prefix E(u) satisfies
E(u) * P >= i * W (W = total cost).

Layout (int32):
  [0] total units U          [1] former size (rows mode, else 0)
  [2] remain size (rows)     [3] remain_num (rows)
  [4] used parts             [5] max key length over batches
  [6] parts P                [7] mode (0 weighted, 1 rows)
  [8] error flags            [9] per-unit overhead (weighted)
  [10..15] 0                 [16 + i] start unit of part i, i = 0..P
"""
from __future__ import annotations

import numpy as np

HEADER = 16
MAX_PARTS = 2048
METADATA_INTS = 2080          # HEADER + MAX_PARTS + 1, rounded up to 16
MODE_WEIGHTED = 0
MODE_ROWS = 1
ERR_CU_Q = 1
ERR_CU_K = 2
ERR_INDEX = 4


def _side_table(layout, n_batch, s, total, cu):
    """Per-batch (start, length) plus an error flag for a bad cu_seqlens."""
    if layout == "BSND":
        return [(b * s, s) for b in range(n_batch)], False
    cu = np.asarray(cu, dtype=np.int64)
    bad = bool(cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != total)
    return [(int(cu[b]), int(cu[b + 1] - cu[b])) for b in range(n_batch)], bad


def metadata_ref(*, layout_q, layout_k, batch, s1, s2, n2, topk, parts, mode,
                 overhead=64, cu_seqlens_q=None, cu_seqlens_k=None,
                 sparse_indices=None, max_seqlen_k=None):
    """Expected metadata array (int32, METADATA_INTS long).

    s1 / s2 are S1 / S2 for BSND sides and the totals T1 / T2 for TND sides.
    ``sparse_indices`` ([T1, N2, topk] flattened rows) is needed in weighted mode.
    """
    if not 1 <= parts <= MAX_PARTS:
        raise ValueError("parts out of range")
    t1 = batch * s1 if layout_q == "BSND" else s1
    t2 = batch * s2 if layout_k == "BSND" else s2
    qtab, bad_q = _side_table(layout_q, batch, s1, t1, cu_seqlens_q)
    ktab, bad_k = _side_table(layout_k, batch, s2, t2, cu_seqlens_k)
    U = t1 * n2
    md = np.zeros(METADATA_INTS, dtype=np.int64)
    md[0] = U
    md[5] = max([kl for _, kl in ktab], default=0) if max_seqlen_k is None else max_seqlen_k
    md[6] = parts
    md[7] = mode
    flags = (ERR_CU_Q if bad_q else 0) | (ERR_CU_K if bad_k else 0)
    bounds = np.zeros(parts + 1, dtype=np.int64)

    if mode == MODE_ROWS:
        if U > 0:
            former = -(-U // parts)
            remain = former - 1
            remain_num = parts * former - U
            former_num = parts - remain_num
            md[1], md[2], md[3] = former, remain, remain_num
            for i in range(parts + 1):
                if i <= former_num:
                    bounds[i] = i * former
                else:
                    bounds[i] = former_num * former + (i - former_num) * remain
    elif mode == MODE_WEIGHTED:
        md[9] = overhead
        idx = np.asarray(sparse_indices, dtype=np.int64).reshape(t1, n2, topk)
        cost = np.zeros(U, dtype=np.int64)
        for b, (q0, qlen) in enumerate(qtab):
            klen = ktab[b][1]
            for t in range(qlen):
                r = q0 + t
                if r < 0 or r >= t1:
                    continue
                for g in range(n2):
                    ids = idx[r, g]
                    ok = (ids >= 0) & (ids < klen)
                    if np.any((ids != -1) & ~ok):
                        flags |= ERR_INDEX
                    cost[r * n2 + g] = int(ok.sum())
        cost += overhead
        excl = np.concatenate([[0], np.cumsum(cost)])        # E(0..U)
        W = int(excl[-1])
        for i in range(parts + 1):
            # first u in [0, U] with E(u) * P >= i * W
            u = 0
            while u < U and excl[u] * parts < i * W:
                u += 1
            bounds[i] = u
    else:
        raise ValueError("unknown mode")

    md[8] = flags
    md[HEADER:HEADER + parts + 1] = bounds
    md[4] = int(np.sum(np.diff(bounds) > 0))
    return md.astype(np.int32)
