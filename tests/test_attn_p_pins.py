"""Pins of the fp64 oracle of p (attnSoftmaxL1Norm): what the operator page and
mathematics fix about "the main attention score summed over heads and
L1-normalised" (readings P1-P4 in oracle/attn_p_ref.py).

* a hand example with closed-form values;
* one head and the slots' own log-sum-exp: p is the textbook softmax of the
  scaled scores (scipy);
* the log-sum-exp of a dense main attention over every key of the batch: p equals
  that attention's probabilities, brute-forced over all keys, taken at the top-k
  slots, summed over heads and L1-normalised;
* invariants: rows sum to 1, 0 at -1 slots, head order, slot order, -1
  insertion, duplicate slots share equally, N2 groups split into separate
  problems, the head-mean closed form;
* planted mistakes in a copy of the unit step, each caught by the pins above.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import attn_p_ref
from oracle.attn_p_ref import attn_p_unit, attn_softmax_l1norm_ref, lse_over_slots_ref


def _problem(seed=0, B=2, S1=6, S2=9, nm=4, n2=1, dm=8, topk=5, invalid=0.2, dups=False):
    rng = np.random.default_rng(seed)
    qm = rng.normal(size=(B, S1, nm, dm))
    km = rng.normal(size=(B, S2, n2, dm))
    idx = np.full((B, S1, n2, topk), -1, dtype=np.int64)
    for b in range(B):
        for t in range(S1):
            for g in range(n2):
                n = int(round((1 - invalid) * topk))
                vals = rng.integers(0, S2, size=n) if dups else rng.choice(S2, size=n, replace=False)
                slots = rng.choice(topk, size=n, replace=False)
                idx[b, t, g, slots] = vals
    return qm, km, idx


def test_hand_example():
    # one head, scale 1/2: z = (1, 0)
    qm = np.array([[[[1.0, 0.0]]]])
    km = np.array([[[[2.0, 0.0]], [[0.0, 1.0]]]])
    idx = np.array([[[[0, 1]]]])
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=0.5)
    e = math.e
    np.testing.assert_allclose(p[0, 0, 0], [e / (e + 1), 1 / (e + 1)], rtol=1e-15)


def test_one_head_is_the_softmax_of_the_scaled_scores():
    qm, km, idx = _problem(seed=1, nm=1, invalid=0.3)
    scale = 0.37
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=scale)
    for b in range(2):
        for t in range(6):
            ids = idx[b, t, 0]
            v = ids >= 0
            z = scale * (km[b, ids[v], 0] @ qm[b, t, 0])
            np.testing.assert_allclose(p[b, t, 0, v], softmax(z), rtol=1e-13)
            assert np.all(p[b, t, 0, ~v] == 0)


def test_dense_log_sum_exp_gives_the_restricted_dense_attention():
    """lse of a dense main attention over all keys of the batch: p is the dense
    probabilities (brute force over every key) at the top-k slots, summed over the
    heads and L1-normalised."""
    qm, km, idx = _problem(seed=2, nm=3, dups=True, invalid=0.4)
    scale = 0.5
    B, S1, nm, dm = qm.shape
    lse = np.zeros((B, S1, nm))
    P_dense = np.zeros((B, S1, nm, km.shape[1]))
    for b in range(B):
        for t in range(S1):
            z_all = scale * (qm[b, t] @ km[b, :, 0].T)        # [nm, S2]
            P_dense[b, t] = softmax(z_all, axis=1)
            lse[b, t] = np.log(np.exp(z_all).sum(axis=1))
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=scale, lse=lse)
    for b in range(B):
        for t in range(S1):
            ids = idx[b, t, 0]
            v = ids >= 0
            a = P_dense[b, t][:, ids[v]].sum(axis=0)
            np.testing.assert_allclose(p[b, t, 0, v], a / a.sum(), rtol=1e-12)


def test_slot_log_sum_exp_given_equals_computed():
    qm, km, idx = _problem(seed=3, nm=4)
    lse = lse_over_slots_ref(qm, km, idx, scale=0.3)
    a = attn_softmax_l1norm_ref(qm, km, idx, scale=0.3)
    b = attn_softmax_l1norm_ref(qm, km, idx, scale=0.3, lse=lse)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-16)


def test_head_mean_closed_form():
    """With the slots' own log-sum-exp every head's probabilities sum to 1 over the
    slots, so the L1 normalisation divides by the head count: p is the head mean
    of the per-head softmaxes."""
    qm, km, idx = _problem(seed=4, nm=3, invalid=0.0)
    scale = 0.7
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=scale)
    for b in range(2):
        for t in range(6):
            ids = idx[b, t, 0]
            z = scale * (qm[b, t] @ km[b, ids, 0].T)
            np.testing.assert_allclose(p[b, t, 0], softmax(z, axis=1).mean(axis=0), rtol=1e-13)


def test_rows_sum_to_one_and_zero_at_padding():
    qm, km, idx = _problem(seed=5, nm=4, invalid=0.5, dups=True)
    idx[0, 2] = -1                                   # a row without a valid slot
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=0.2)
    valid = idx >= 0
    assert np.all(p[~valid] == 0)
    sums = p.sum(-1)
    np.testing.assert_allclose(sums[valid.any(-1)], 1.0, rtol=1e-14)
    assert np.all(p[0, 2] == 0)


def test_head_order_slot_order_and_padding_invariance():
    qm, km, idx = _problem(seed=6, nm=4, invalid=0.2)
    base = attn_softmax_l1norm_ref(qm, km, idx, scale=0.4)
    hp = np.random.default_rng(0).permutation(4)
    assert np.allclose(attn_softmax_l1norm_ref(qm[:, :, hp], km, idx, scale=0.4), base, rtol=1e-13, atol=0)
    sp = np.random.default_rng(1).permutation(idx.shape[-1])
    np.testing.assert_allclose(attn_softmax_l1norm_ref(qm, km, idx[..., sp], scale=0.4), base[..., sp],
                               rtol=1e-13)
    pad = np.concatenate([idx, np.full(idx.shape[:-1] + (3,), -1)], axis=-1)
    got = attn_softmax_l1norm_ref(qm, km, pad, scale=0.4)
    np.testing.assert_allclose(got[..., :idx.shape[-1]], base, rtol=1e-13)
    assert np.all(got[..., idx.shape[-1]:] == 0)


def test_duplicate_slots_share_equally():
    qm, km, idx = _problem(seed=7, nm=2, invalid=0.0)
    idx[1, 3, 0, 1] = idx[1, 3, 0, 0]
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=0.5)
    assert p[1, 3, 0, 0] == p[1, 3, 0, 1]
    assert p.sum(-1)[1, 3, 0] == pytest.approx(1.0, rel=1e-14)


def test_key_heads_split_into_separate_problems():
    """N2 = 2: key head g owns main-attention heads g Hm .. (g+1) Hm - 1 (reading P3)."""
    qm, km, idx = _problem(seed=8, nm=6, n2=2)
    p = attn_softmax_l1norm_ref(qm, km, idx, scale=0.3)
    for g in range(2):
        pg = attn_softmax_l1norm_ref(qm[:, :, 3 * g:3 * g + 3], km[:, :, g:g + 1], idx[:, :, g:g + 1], scale=0.3)
        np.testing.assert_allclose(p[:, :, g:g + 1], pg, rtol=1e-14)


def test_bsnd_equals_tnd():
    qm, km, idx = _problem(seed=9, nm=2)
    a = attn_softmax_l1norm_ref(qm, km, idx, scale=0.3)
    cu_q = np.array([0, 6, 12])
    cu_k = np.array([0, 9, 18])
    b = attn_softmax_l1norm_ref(qm.reshape(12, 2, 8), km.reshape(18, 1, 8), idx.reshape(12, 1, 5), scale=0.3,
                                layout_q="TND", layout_k="TND", cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    np.testing.assert_allclose(a.reshape(b.shape), b, rtol=1e-14)


def test_out_of_range_index_raises():
    qm, km, idx = _problem(seed=10)
    idx[0, 0, 0, 0] = 9
    with pytest.raises(ValueError):
        attn_softmax_l1norm_ref(qm, km, idx, scale=0.3)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the unit step must fail a pin above.
# ---------------------------------------------------------------------------
def _mutant(kind):
    def unit(qm_t, km_sel, valid, scale, lse_t=None):
        K = km_sel.shape[0]
        p = np.zeros(K)
        v = np.flatnonzero(valid)
        if v.size == 0:
            return p
        z = (1.0 if kind == "no_scale" else scale) * (qm_t @ km_sel[v].T)
        if lse_t is None:
            lse = np.log(np.exp(z).sum(axis=1))
        else:
            lse = np.asarray(lse_t)
        if kind == "lse_sign":
            lse = -lse
        P = np.exp(z - lse[:, None])
        a = P[0] if kind == "first_head" else P.sum(axis=0)
        if kind == "max_heads":
            a = P.max(axis=0)
        p[v] = a / (a.sum() if kind != "no_norm" else 1.0)
        return p
    return unit


@pytest.mark.parametrize("kind", ["no_scale", "lse_sign", "first_head", "max_heads", "no_norm"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(attn_p_ref, "attn_p_unit", _mutant(kind))
    pins = [test_hand_example, test_one_head_is_the_softmax_of_the_scaled_scores,
            test_dense_log_sum_exp_gives_the_restricted_dense_attention, test_head_mean_closed_form]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, kind
