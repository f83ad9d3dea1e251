"""Pins of the metadata reference (integer split of units over parts).

The split of the rows mode follows the prose of the metadata article's
功能定位 section (CeilDiv into former-size parts, remain = former - 1);
these tests pin it by hand-computed cases and by brute force over the
definition; the weighted mode is pinned by brute force over its definition.
"""
import numpy as np
import pytest

from oracle.metadata_ref import HEADER, MODE_ROWS, MODE_WEIGHTED, metadata_ref


def _rows(U, P):
    return metadata_ref(layout_q="BSND", layout_k="BSND", batch=1, s1=U, s2=4, n2=1,
                        topk=1, parts=P, mode=MODE_ROWS)


@pytest.mark.parametrize("U,P,bounds,hdr", [
    (10, 4, [0, 3, 6, 8, 10], (3, 2, 2, 4)),     # former 3, two parts of 2
    (3, 4, [0, 1, 2, 3, 3], (1, 0, 1, 3)),       # fewer units than parts
    (8, 4, [0, 2, 4, 6, 8], (2, 1, 0, 4)),       # exact split
    (1, 1, [0, 1], (1, 0, 0, 1)),
])
def test_rows_mode_hand_cases(U, P, bounds, hdr):
    md = _rows(U, P)
    assert md[0] == U and md[6] == P and md[7] == MODE_ROWS
    assert tuple(md[1:5]) == hdr
    assert list(md[HEADER:HEADER + P + 1]) == bounds


@pytest.mark.parametrize("U", [1, 5, 17, 255, 256, 257, 1000])
@pytest.mark.parametrize("P", [1, 7, 256])
def test_rows_mode_structure(U, P):
    md = _rows(U, P)
    b = md[HEADER:HEADER + P + 1].astype(np.int64)
    sizes = np.diff(b)
    assert b[0] == 0 and b[-1] == U and np.all(sizes >= 0)
    former, remain = md[1], md[2]
    assert set(sizes.tolist()) <= {former, remain}
    assert former == -(-U // P)
    # larger shares come first
    assert np.all(np.diff(sizes) <= 0)
    assert md[4] == int(np.sum(sizes > 0))


def test_weighted_mode_brute_force():
    rng = np.random.default_rng(0)
    T1, n2, topk = 37, 2, 9
    idx = rng.integers(-1, 5, size=(T1, n2, topk)).astype(np.int32)
    for P in (1, 3, 16, 100):
        md = metadata_ref(layout_q="BSND", layout_k="BSND", batch=1, s1=T1, s2=5, n2=n2,
                          topk=topk, parts=P, mode=MODE_WEIGHTED, overhead=3,
                          sparse_indices=idx)
        cost = (idx >= 0).sum(-1).reshape(-1) + 3
        E = np.concatenate([[0], np.cumsum(cost)])
        W = E[-1]
        b = md[HEADER:HEADER + P + 1]
        for i in range(P + 1):
            cand = [u for u in range(len(cost) + 1) if E[u] * P >= i * W]
            assert b[i] == min(cand)
        # every part's cost is within one unit's cost of W / P
        part_cost = E[b[1:]] - E[b[:-1]]
        assert np.all(part_cost <= W / P + cost.max())
        assert md[8] == 0


def test_weighted_mode_flags_out_of_range_and_bad_cu():
    idx = np.array([[[0, 7, -1]], [[1, -1, -1]]], dtype=np.int32)   # 7 >= key length 5
    md = metadata_ref(layout_q="TND", layout_k="TND", batch=1, s1=2, s2=4, n2=1, topk=3,
                      parts=2, mode=MODE_WEIGHTED, overhead=1,
                      cu_seqlens_q=np.array([0, 2]), cu_seqlens_k=np.array([0, 5]),
                      sparse_indices=idx)
    assert md[8] & 4          # index out of the batch's key range
    assert md[8] & 2          # cu_seqlens_k does not end at the key total
    assert not md[8] & 1
