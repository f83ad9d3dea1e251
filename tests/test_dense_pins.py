"""Pins of the fp64 oracle of the dense sibling operator (oracle/dense_ref.py).

The metadata article fixes the mask modes of the dense operator (0: none, 3:
rightDownCausal, the lower triangle cornered at the bottom-right vertex); the
formulas are the sparse operator's with the top-k set replaced by the visible keys
(reading D1).  Pinned by:

* the mask written out by hand for a small S1 < S2, S1 = S2 and S1 > S2 case;
* fp64 torch autograd of the dense KL loss with an explicit mask matrix;
* the sparse oracle (pinned on its own) given index lists of the visible keys;
* closed forms: the first row under mask 3 with S1 = S2 sees one key (y = 1, and
  p = 1 there gives zero gradients); rows that see nothing are zero;
* BSND equals TND; planted mistakes in the mask rule.
"""
import numpy as np
import pytest

from oracle import dense_ref
from oracle.dense_ref import dense_grad_ref, visible_keys
from oracle.slikl_ref import slikl_grad_ref


def _problem(seed=0, B=2, S1=5, S2=7, n1=4, n2=1, d=6, peaky=False):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, S1, n1, d))
    k = rng.normal(size=(B, S2, n2, d))
    w = rng.normal(scale=0.7, size=(B, S1, n1))
    logits = rng.normal(scale=2.0 if peaky else 1.0, size=(B, S1, n2, S2))
    return q, k, w, logits


def _p_for(logits, mask_mode, S1, S2):
    """Target distribution over each row's visible keys (0 elsewhere)."""
    p = np.zeros_like(logits)
    for t in range(S1):
        n = visible_keys(mask_mode, t, S1, S2)
        if n:
            e = np.exp(logits[:, t, :, :n] - logits[:, t, :, :n].max(-1, keepdims=True))
            p[:, t, :, :n] = e / e.sum(-1, keepdims=True)
    return p


def test_mask_by_hand():
    # rightDownCausal: rows and keys aligned at the bottom-right corner
    got = np.array([[1 if j < visible_keys(3, t, 3, 5) else 0 for j in range(5)] for t in range(3)])
    want = np.array([[1, 1, 1, 0, 0],
                     [1, 1, 1, 1, 0],
                     [1, 1, 1, 1, 1]])
    assert np.array_equal(got, want)
    got = np.array([[1 if j < visible_keys(3, t, 4, 4) else 0 for j in range(4)] for t in range(4)])
    assert np.array_equal(got, np.tril(np.ones((4, 4), dtype=int)))
    got = np.array([[1 if j < visible_keys(3, t, 5, 2) else 0 for j in range(2)] for t in range(5)])
    want = np.array([[0, 0], [0, 0], [0, 0], [1, 0], [1, 1]])
    assert np.array_equal(got, want)
    assert all(visible_keys(0, t, 5, 2) == 2 for t in range(5))


@pytest.mark.parametrize("mask_mode,S1,S2", [(3, 5, 7), (3, 6, 6), (3, 6, 4), (0, 4, 6)])
def test_autograd_of_the_dense_kl_loss(torch_cpu, mask_mode, S1, S2):
    torch = torch_cpu
    q, k, w, logits = _problem(seed=S1 * 10 + S2, S1=S1, S2=S2, n1=4, n2=2, d=5)
    p = _p_for(logits, mask_mode, S1, S2)
    ref = dense_grad_ref(q, k, w, p, mask_mode=mask_mode)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    G = 2
    vis = torch.tensor([[j < visible_keys(mask_mode, t, S1, S2) for j in range(S2)] for t in range(S1)])
    loss = torch.zeros((), dtype=torch.float64)
    ys = np.zeros_like(p)
    for b in range(q.shape[0]):
        for g in range(2):
            S = torch.einsum("thd,jd->thj", qt[b, :, g * G:(g + 1) * G], kt[b, :, g])   # [S1, G, S2]
            I = torch.einsum("th,thj->tj", wt[b, :, g * G:(g + 1) * G], torch.relu(S))
            I = I.masked_fill(~vis, float("-inf"))
            for t in range(S1):
                if not vis[t].any():
                    continue
                logy = torch.log_softmax(I[t][vis[t]], dim=0)
                pt = torch.tensor(p[b, t, g][vis[t].numpy()])
                nz = pt > 0
                loss = loss + torch.sum(pt[nz] * (torch.log(pt[nz]) - logy[nz]))
                ys[b, t, g, vis[t].numpy()] = torch.exp(logy).detach().numpy()
    loss.backward()
    np.testing.assert_allclose(ref["softmax_out"], ys, atol=1e-14)
    np.testing.assert_allclose(ref["dq"], qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(ref["dk"], kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(ref["dw"], wt.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("mask_mode", [0, 3])
def test_equals_the_sparse_oracle_on_the_visible_keys(mask_mode):
    q, k, w, logits = _problem(seed=3, S1=6, S2=8, n1=6, n2=2, d=4)
    p = _p_for(logits, mask_mode, 6, 8)
    idx = np.full(p.shape, -1, dtype=np.int64)
    for t in range(6):
        n = visible_keys(mask_mode, t, 6, 8)
        idx[:, t, :, :n] = np.arange(n)
    a = dense_grad_ref(q, k, w, p, mask_mode=mask_mode)
    b = slikl_grad_ref(q, k, w, idx, p)
    for name in ("dq", "dk", "dw", "softmax_out"):
        np.testing.assert_allclose(a[name], b[name], rtol=1e-12, atol=1e-14)


def test_first_row_sees_one_key():
    q, k, w, logits = _problem(seed=4, S1=4, S2=4)
    p = _p_for(logits, 3, 4, 4)
    ref = dense_grad_ref(q, k, w, p, mask_mode=3)
    assert np.all(ref["softmax_out"][:, 0, :, 0] == 1.0)
    assert np.all(ref["softmax_out"][:, 0, :, 1:] == 0.0)
    # p = 1 on the one key: y = p, so the row's gradients vanish
    assert np.all(ref["dq"][:, 0] == 0) and np.all(ref["dw"][:, 0] == 0)


def test_rows_that_see_nothing_are_zero():
    q, k, w, logits = _problem(seed=5, S1=6, S2=3)
    p = _p_for(logits, 3, 6, 3)
    ref = dense_grad_ref(q, k, w, p, mask_mode=3)
    for t in range(3):                              # rows 0..2 see no key
        assert np.all(ref["dq"][:, t] == 0) and np.all(ref["softmax_out"][:, t] == 0)
    assert np.abs(ref["dq"][:, 3:]).max() > 0


def test_bsnd_equals_tnd():
    q, k, w, logits = _problem(seed=6, B=2, S1=5, S2=7)
    p = _p_for(logits, 3, 5, 7)
    a = dense_grad_ref(q, k, w, p, mask_mode=3)
    b = dense_grad_ref(q.reshape(10, 4, 6), k.reshape(14, 1, 6), w.reshape(10, 4), p.reshape(10, 1, 7),
                       mask_mode=3, layout_q="TND", layout_k="TND", cu_seqlens_q=np.array([0, 5, 10]),
                       cu_seqlens_k=np.array([0, 7, 14]))
    for name in ("dq", "dk", "dw", "softmax_out"):
        np.testing.assert_allclose(a[name].reshape(b[name].shape), b[name], rtol=1e-14)


@pytest.mark.parametrize("kind", ["top_left", "strict", "no_mask"])
def test_planted_mask_mistakes_are_caught(torch_cpu, monkeypatch, kind):
    """A wrong mask rule inside the oracle fails the autograd pin (whose mask comes
    from the rule pinned by hand above)."""
    def wrong(mask_mode, t, s1_b, s2_b):
        if kind == "top_left":
            return min(s2_b, t + 1) if mask_mode == 3 else s2_b
        if kind == "strict":
            return int(max(0, min(s2_b, t + (s2_b - s1_b)))) if mask_mode == 3 else s2_b
        return s2_b
    monkeypatch.setattr(dense_ref, "visible_keys", wrong)
    with pytest.raises(AssertionError):
        test_autograd_of_the_dense_kl_loss(torch_cpu, 3, 5, 7)
