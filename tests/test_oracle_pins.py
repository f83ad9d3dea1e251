"""Pins of the fp64 oracle against what the operator page and mathematics fix.

The operator page ("aclnnSparseLightningIndexerKLLossGrad", formula section)
defines the forward quantities (S, I, y = Softmax(I), the KL loss) and states
the gradients.  The page prints no worked example with values, so the oracle
is pinned by:

* a hand-derived closed-form example (one head, D = 1, two keys);
* torch fp64 autograd of the KL loss written in a different formulation
  (one-hot selection matrices instead of index gathers), including duplicate
  indices, -1 padding, N2 = 2 groups and the TND layout;
* central finite differences of the loss;
* special cases with closed forms (w = 0, p = y, a single valid slot);
* invariants (softmax rows sum to 1, slot-order and -1-insertion invariance,
  BSND == TND on the same data, the literal dI = y - p reading).

A final group plants mistakes in a copy of the oracle's unit step and checks
that the autograd pin catches each of them.
"""
import math

import numpy as np
import pytest

from oracle import slikl_ref
from oracle.slikl_ref import kl_loss_ref, kl_per_unit_ref, slikl_grad_ref, unit_backward
from workloads import Workload, make_inputs


def _small(seed=0, **kw):
    base = dict(name="pin", layout="BSND", batch=2, s1=7, s2=9, n1=4, n2=1, d=5, topk=6,
                dtype="bf16", w_var=0.5, index_mode="random", invalid_frac=0.2,
                p_var=1.0, seed=seed)
    base.update(kw)
    return make_inputs(Workload(**base))


def _args(x):
    return dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=x.cu_q,
                cu_seqlens_k=x.cu_k)


# ---------------------------------------------------------------------------
# Independent formulation: one-hot selection matrices + torch autograd (fp64).
# ---------------------------------------------------------------------------
def _torch_loss_and_grads(torch, x):
    """KL loss through dense one-hot selection; returns (L, dq, dk, dw, y).  The
    per-unit terms of L are left in x.kl_units ([T1, N2])."""
    q = torch.tensor(x.q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(x.k, dtype=torch.float64, requires_grad=True)
    w = torch.tensor(x.w, dtype=torch.float64, requires_grad=True)
    n1, d = x.q.shape[-2:]
    n2 = x.k.shape[-2]
    G = n1 // n2
    topk = x.idx.shape[-1]
    qf, kf, wf = q.reshape(-1, n1, d), k.reshape(-1, n2, d), w.reshape(-1, n1)
    idx = x.idx.reshape(-1, n2, topk)
    p = x.p.reshape(-1, n2, topk).astype(np.float64)
    T2 = kf.shape[0]
    if x.layout_q == "BSND":
        B, S1 = x.q.shape[0], x.q.shape[1]
        qstart = [b * S1 for b in range(B)] + [B * S1]
    else:
        qstart = [int(c) for c in x.cu_q]
    if x.layout_k == "BSND":
        S2 = x.k.shape[1]
        kstart = [b * S2 for b in range(len(qstart) - 1)]
    else:
        kstart = [int(c) for c in x.cu_k[:-1]]
    loss = torch.zeros((), dtype=torch.float64)
    ys = np.zeros(idx.shape)
    units = np.zeros(idx.shape[:2])
    for b in range(len(qstart) - 1):
        for r in range(qstart[b], qstart[b + 1]):
            for g in range(n2):
                sel = np.zeros((topk, T2))
                valid = idx[r, g] >= 0
                for s in range(topk):
                    if valid[s]:
                        sel[s, kstart[b] + idx[r, g, s]] = 1.0
                if not valid.any():
                    continue
                Sel = torch.tensor(sel[valid])
                Ksel = Sel @ kf[:, g, :]                          # [|V|, D]
                S = qf[r, g * G:(g + 1) * G] @ Ksel.T            # [G, |V|]
                I = wf[r, g * G:(g + 1) * G] @ torch.relu(S)
                logy = torch.log_softmax(I, dim=0)
                pv = torch.tensor(p[r, g, valid])
                nz = pv > 0
                term = torch.sum(pv[nz] * (torch.log(pv[nz]) - logy[nz]))
                units[r, g] = float(term.detach())
                loss = loss + term
                ys[r, g, valid] = torch.exp(logy).detach().numpy()
    loss.backward()
    x.kl_units = units
    return (float(loss.detach()), q.grad.numpy(), k.grad.numpy(), w.grad.numpy(),
            ys.reshape(x.p.shape))


def _normalise_p(x):
    """Make p sum to 1 over each row's valid slots (KL gradient = y - p then)."""
    p = x.p.astype(np.float64)
    s = p.sum(axis=-1, keepdims=True)
    x.p = np.where(s > 0, p / np.where(s > 0, s, 1), 0).astype(np.float64)
    return x


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)


CASES = [
    dict(),                                                       # BSND, -1 padding
    dict(index_mode="random", duplicates=True, invalid_frac=0.3),  # duplicate indices
    dict(n1=6, n2=2, d=3),                                        # two key heads
    dict(layout="TND", batch=3, seqlens=(5, 1, 8), s1=0, s2=0),   # varlen TND
    dict(index_mode="causal", s1=8, s2=8, topk=5),                # causal, trailing -1
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_autograd_matches(torch_cpu, case):
    x = _normalise_p(_small(seed=10 + case, **CASES[case]))
    ref = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    L, dq, dk, dw, y = _torch_loss_and_grads(torch_cpu, x)
    assert _rel(ref["dq"], dq) < 1e-10
    assert _rel(ref["dk"], dk) < 1e-10
    assert _rel(ref["dw"], dw) < 1e-10
    assert np.max(np.abs(ref["softmax_out"] - y)) < 1e-12
    assert abs(kl_loss_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x)) - L) < 1e-10 * max(1, abs(L))
    units = kl_per_unit_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    assert np.max(np.abs(units - x.kl_units)) < 1e-10 * max(1, np.max(np.abs(x.kl_units)))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_kl_per_unit_closed_forms(case):
    """KL(p || Softmax(I)) per unit: 0 when p is the unit's softmax itself, -log y_s
    when p is one-hot at slot s, 0 for a unit without a valid slot; the units sum to
    the total loss."""
    x = _small(seed=30 + case, **CASES[case])
    args = _args(x)
    y = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **args)["softmax_out"]
    valid = x.idx >= 0
    same = kl_per_unit_ref(x.q, x.k, x.w, x.idx, y, **args)
    assert np.max(np.abs(same)) < 1e-12
    first = np.argmax(valid, axis=-1)[..., None]                 # first valid slot per unit
    onehot = np.zeros_like(y)
    np.put_along_axis(onehot, first, 1.0, axis=-1)
    onehot = np.where(valid.any(-1, keepdims=True), onehot, 0.0)
    got = kl_per_unit_ref(x.q, x.k, x.w, x.idx, onehot, **args)
    ys = np.take_along_axis(y, first, axis=-1)[..., 0]
    want = np.where(valid.any(-1), -np.log(np.where(valid.any(-1), ys, 1.0)), 0.0)
    assert np.max(np.abs(got.reshape(want.shape) - want)) < 1e-12 * max(1, np.max(np.abs(want)))
    tot = kl_loss_ref(x.q, x.k, x.w, x.idx, x.p, **args)
    assert abs(kl_per_unit_ref(x.q, x.k, x.w, x.idx, x.p, **args).sum() - tot) < 1e-10 * max(1, abs(tot))


def test_finite_differences():
    """Central differences of L pin dq, dk and dw (fp64, h = 1e-6)."""
    rng = np.random.default_rng(7)
    for attempt in range(50):
        x = _normalise_p(_small(seed=100 + attempt, batch=1, s1=6, s2=6, n1=3, d=4,
                                topk=4, invalid_frac=0.25))
        # keep away from ReLU kinks: every |S| over valid pairs must exceed 1e-3
        qf, kf = x.q.reshape(-1, 3, 4).astype(np.float64), x.k.reshape(-1, 1, 4).astype(np.float64)
        idx = x.idx.reshape(-1, 1, 4)
        S = [qf[r] @ kf[idx[r, 0, s], 0] for r in range(6) for s in range(4) if idx[r, 0, s] >= 0]
        if min(np.min(np.abs(v)) for v in S) > 1e-3:
            break
    else:
        pytest.fail("no kink-free draw")
    args = _args(x)
    ref = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **args)
    h = 1e-6
    for name in ("q", "k", "w"):
        base = getattr(x, name).astype(np.float64)
        grad = np.zeros_like(base)
        for i in range(base.size):
            plus, minus = base.copy(), base.copy()
            plus.flat[i] += h
            minus.flat[i] -= h
            kw = {"q": x.q, "k": x.k, "w": x.w}
            kw[name] = plus
            lp = kl_loss_ref(kw["q"], kw["k"], kw["w"], x.idx, x.p, **args)
            kw[name] = minus
            lm = kl_loss_ref(kw["q"], kw["k"], kw["w"], x.idx, x.p, **args)
            grad.flat[i] = (lp - lm) / (2 * h)
        want = ref["d" + name]
        err = np.max(np.abs(grad - want)) / max(np.max(np.abs(want)), 1e-12)
        assert err < 1e-6, (name, err)
    del rng


def test_hand_example():
    """One head, D = 1, q = 1, keys 1 and 2, w = 1, p = (1/2, 1/2).

    S = (1, 2), I = (1, 2), y = (1, e) / (1 + e), dI = y - 1/2,
    dw = dI . (1, 2), dq = dI . (1, 2), dk_j = dI_j * q.
    """
    q = np.array([[[[1.0]]]])
    k = np.array([[[[1.0]], [[2.0]]]])
    w = np.array([[[1.0]]])
    idx = np.array([[[[0, 1]]]], dtype=np.int32)
    p = np.array([[[[0.5, 0.5]]]])
    out = slikl_grad_ref(q, k, w, idx, p)
    e = math.e
    y = np.array([1 / (1 + e), e / (1 + e)])
    dI = y - 0.5
    assert np.allclose(out["softmax_out"].ravel(), y, rtol=0, atol=1e-15)
    assert abs(out["dw"].item() - (dI[0] + 2 * dI[1])) < 1e-15
    assert abs(out["dq"].item() - (dI[0] * 1 + dI[1] * 2)) < 1e-15
    assert np.allclose(out["dk"].ravel(), dI, rtol=0, atol=1e-15)


def test_hand_example_negative_score():
    """A key with S < 0 is masked out of dq / dk / dw but still in the softmax."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[-1.0]], [[2.0]]]])
    w = np.array([[[0.5]]])
    idx = np.array([[[[0, 1]]]], dtype=np.int32)
    p = np.array([[[[0.25, 0.75]]]])
    out = slikl_grad_ref(q, k, w, idx, p)
    # S = (-1, 2), R = (0, 2), I = (0, 1), y = (1, e) / (1 + e)
    e = math.e
    y = np.array([1 / (1 + e), e / (1 + e)])
    dI = y - np.array([0.25, 0.75])
    assert np.allclose(out["softmax_out"].ravel(), y, atol=1e-15)
    assert abs(out["dw"].item() - 2 * dI[1]) < 1e-15               # dW = dI . R
    assert abs(out["dq"].item() - 0.5 * dI[1] * 2.0) < 1e-15       # only key 1 passes
    assert np.allclose(out["dk"].ravel(), [0.0, 0.5 * dI[1] * 1.0], atol=1e-15)


def test_softmax_rows_sum_to_one():
    x = _small(seed=3, batch=3, s1=10, s2=10, topk=8, invalid_frac=0.4)
    y = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))["softmax_out"]
    valid = x.idx >= 0
    assert np.all(y[~valid] == 0)
    sums = y.sum(-1)
    has = valid.any(-1)
    assert np.all(np.abs(sums[has] - 1) < 1e-12)
    assert np.all(sums[~has] == 0)


def test_zero_weights_closed_form():
    """w = 0: I = 0, y = 1/|V|, dq = dk = 0, dw[h] = sum_s (1/|V| - p_s) ReLU(S[h,s])."""
    x = _small(seed=4)
    x.w = np.zeros_like(x.w)
    out = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    assert np.all(out["dq"] == 0) and np.all(out["dk"] == 0)
    B, S1, N1, D = x.q.shape
    for b in range(B):
        for t in range(S1):
            ids = x.idx[b, t, 0]
            v = [s for s in range(len(ids)) if ids[s] >= 0]
            for s in range(len(ids)):
                want = 1.0 / len(v) if s in v else 0.0
                assert abs(out["softmax_out"][b, t, 0, s] - want) < 1e-15
            for h in range(N1):
                acc = 0.0
                for s in v:
                    sc = sum(float(x.q[b, t, h, i]) * float(x.k[b, ids[s], 0, i]) for i in range(D))
                    acc += (1.0 / len(v) - float(x.p[b, t, 0, s])) * max(sc, 0.0)
                assert abs(out["dw"][b, t, h] - acc) < 1e-12


def test_target_equal_softmax_gives_zero_gradients():
    x = _small(seed=5)
    first = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    out = slikl_grad_ref(x.q, x.k, x.w, x.idx, first["softmax_out"], **_args(x))
    for name in ("dq", "dk", "dw"):
        assert np.max(np.abs(out[name])) < 1e-13


def test_single_valid_slot():
    x = _small(seed=6, topk=5, invalid_frac=0.0)
    x.idx[..., 0] = 0
    x.idx[..., 1:] = -1
    x.p = np.zeros_like(x.p)
    x.p[..., 0] = 1.0
    out = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    assert np.all(out["softmax_out"][..., 0] == 1.0)
    for name in ("dq", "dk", "dw"):
        assert np.max(np.abs(out[name])) == 0


def test_slot_permutation_invariance():
    x = _small(seed=8, batch=2, s1=6, s2=7, topk=7, invalid_frac=0.3)
    a = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    perm = np.random.default_rng(1).permutation(x.idx.shape[-1])
    b = slikl_grad_ref(x.q, x.k, x.w, x.idx[..., perm], x.p[..., perm], **_args(x))
    for name in ("dq", "dk", "dw"):
        assert _rel(b[name], a[name]) < 1e-13
    assert np.max(np.abs(b["softmax_out"] - a["softmax_out"][..., perm])) < 1e-15


def test_minus_one_insertion_invariance():
    x = _small(seed=9, topk=5, invalid_frac=0.0)
    a = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    pad = np.full(x.idx.shape[:-1] + (3,), -1, dtype=np.int32)
    idx2 = np.concatenate([pad[..., :1], x.idx[..., :2], pad[..., 1:], x.idx[..., 2:]], -1)
    junk = np.random.default_rng(2).random(pad.shape)          # p at -1 slots is ignored
    p2 = np.concatenate([junk[..., :1], x.p[..., :2], junk[..., 1:], x.p[..., 2:]], -1)
    b = slikl_grad_ref(x.q, x.k, x.w, idx2, p2, **_args(x))
    for name in ("dq", "dk", "dw"):
        assert _rel(b[name], a[name]) < 1e-13
    keep = np.r_[1:3, 5:8]
    assert np.max(np.abs(b["softmax_out"][..., keep] - a["softmax_out"])) < 1e-15
    assert np.all(b["softmax_out"][..., [0, 3, 4]] == 0)


def test_bsnd_equals_tnd():
    x = _small(seed=11, batch=3, s1=5, s2=6)
    a = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    cu_q = np.arange(4, dtype=np.int32) * 5
    cu_k = np.arange(4, dtype=np.int32) * 6
    b = slikl_grad_ref(x.q.reshape(15, *x.q.shape[2:]), x.k.reshape(18, *x.k.shape[2:]),
                       x.w.reshape(15, -1), x.idx.reshape(15, *x.idx.shape[2:]),
                       x.p.reshape(15, *x.p.shape[2:]), layout_q="TND", layout_k="TND",
                       cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    assert np.array_equal(a["dq"].reshape(b["dq"].shape), b["dq"])
    assert np.array_equal(a["dk"].reshape(b["dk"].shape), b["dk"])
    assert np.array_equal(a["dw"].reshape(b["dw"].shape), b["dw"])


def test_literal_di_reading():
    """dI = y - p even when p does not sum to 1: gradients are affine in p."""
    x = _small(seed=12)
    args = _args(x)
    g1 = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **args)
    g2 = slikl_grad_ref(x.q, x.k, x.w, x.idx, 2 * x.p.astype(np.float64), **args)
    g0 = slikl_grad_ref(x.q, x.k, x.w, x.idx, np.zeros_like(x.p), **args)
    for name in ("dq", "dk", "dw"):
        assert _rel(g2[name], 2 * g1[name] - g0[name]) < 1e-12


def test_dk_column_sum_vanishes_when_all_scores_positive():
    """With S > 0 everywhere dS = w dI, and sum_s dI_s = 0 when p sums to 1,
    so the scatter-added dK of one token sums to zero over keys."""
    x = _normalise_p(_small(seed=13, batch=1, s1=1, s2=8, topk=6, invalid_frac=0.0))
    x.q = np.abs(x.q).astype(np.float64)
    x.k = np.abs(x.k).astype(np.float64) + 0.1
    x.idx[0, 0, 0] = np.random.default_rng(3).choice(8, 6, replace=False)
    out = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    assert np.max(np.abs(out["dk"].sum(axis=(0, 1)))) < 1e-13
    assert np.max(np.abs(out["dk"])) > 1e-6


def test_out_of_range_index_raises():
    x = _small(seed=14)
    x.idx[0, 0, 0, 0] = 9
    with pytest.raises(ValueError):
        slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))


# ---------------------------------------------------------------------------
# Planted mistakes: each mutated unit step must fail the autograd pin.
# ---------------------------------------------------------------------------
def _mutant(kind):
    def unit(q_t, k_sel, valid, w_t, p_t, kink=False):
        G, D = q_t.shape
        K = k_sel.shape[0]
        v = np.flatnonzero(valid)
        y = np.zeros(K)
        dk_part = np.zeros((K, D))
        if v.size == 0:
            return y, np.zeros((G, D)), np.zeros(G), dk_part
        kv = k_sel[v]
        S = q_t @ kv.T
        R = np.maximum(S, 0.0)
        I = w_t @ R
        e = np.exp(I - I.max())
        yv = e / e.sum()
        dI = (p_t[v] - yv) if kind == "sign" else (yv - p_t[v])
        dw = R @ dI if kind != "dw_no_relu" else S @ dI
        mask = (S > 0.0) if kind != "no_mask" else 1.0
        dS = w_t[:, None] * dI[None, :] * mask
        dq = dS @ kv
        P = dS.T @ q_t
        if kind == "dk_shift":
            P = np.roll(P, 1, axis=0)
        dk_part[v] = P
        y[v] = yv
        return y, dq, dw, dk_part
    return unit


@pytest.mark.parametrize("kind", ["sign", "dw_no_relu", "no_mask", "dk_shift"])
def test_planted_mistakes_are_caught(torch_cpu, monkeypatch, kind):
    x = _normalise_p(_small(seed=20))
    _, dq, dk, dw, _ = _torch_loss_and_grads(torch_cpu, x)
    monkeypatch.setattr(slikl_ref, "unit_backward", _mutant(kind))
    out = slikl_ref.slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    worst = max(_rel(out["dq"], dq), _rel(out["dk"], dk), _rel(out["dw"], dw))
    assert worst > 1e-3, kind


def test_seq_used_equals_the_cut_problem():
    """seqUsedQ / seqUsedK (TND): the outputs equal those of the problem built from
    each batch's used rows and keys only; the other query rows give 0, the other keys
    get no dK."""
    x = _small(seed=77, layout="TND", batch=3, seqlens=(5, 1, 8), s1=0, s2=0, topk=6)
    used_q = np.array([3, 1, 0])
    used_k = np.array([4, 0, 8])
    cu = x.cu_q.astype(np.int64)
    idx = x.idx.copy()
    for b in range(3):
        rows = slice(cu[b], cu[b + 1])
        idx[rows] = np.where(idx[rows] >= used_k[b], -1, idx[rows])    # inside the used keys
    full = slikl_grad_ref(x.q, x.k, x.w, idx, x.p, layout_q="TND", layout_k="TND",
                          cu_seqlens_q=cu, cu_seqlens_k=cu, seq_used_q=used_q, seq_used_k=used_k)
    qr = np.concatenate([np.arange(cu[b], cu[b] + used_q[b]) for b in range(3)]).astype(int)
    kr = np.concatenate([np.arange(cu[b], cu[b] + used_k[b]) for b in range(3)]).astype(int)
    cuq = np.concatenate([[0], np.cumsum(used_q)])
    cuk = np.concatenate([[0], np.cumsum(used_k)])
    cut = slikl_grad_ref(x.q[qr], x.k[kr], x.w[qr], idx[qr], x.p[qr], layout_q="TND",
                         layout_k="TND", cu_seqlens_q=cuq, cu_seqlens_k=cuk)
    for name in ("dq", "dw", "softmax_out"):
        assert np.array_equal(full[name][qr], cut[name])
        rest = np.setdiff1d(np.arange(full[name].shape[0]), qr)
        assert not np.any(full[name][rest])
    assert np.allclose(full["dk"][kr], cut["dk"], rtol=1e-13, atol=1e-15)
    assert not np.any(np.delete(full["dk"], kr, axis=0))
    units = kl_per_unit_ref(x.q, x.k, x.w, idx, x.p, layout_q="TND", layout_k="TND",
                            cu_seqlens_q=cu, cu_seqlens_k=cu, seq_used_q=used_q, seq_used_k=used_k)
    units_cut = kl_per_unit_ref(x.q[qr], x.k[kr], x.w[qr], idx[qr], x.p[qr], layout_q="TND",
                                layout_k="TND", cu_seqlens_q=cuq, cu_seqlens_k=cuk)
    assert np.allclose(units[qr], units_cut, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Mask decisions at S = 0 (reading 11): the kink allowance.
# ---------------------------------------------------------------------------
def _unit_grads_torch(torch, q_t, k_sel, w_t, p_t, ge):
    """One unit's gradients by fp64 autograd of its KL term, with ReLU written as
    where(S > 0, S, 0) (ge=False: derivative 0 at S = 0) or where(S >= 0, S, 0)
    (ge=True: derivative 1 at S = 0)."""
    q = torch.tensor(q_t, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(k_sel, dtype=torch.float64, requires_grad=True)
    w = torch.tensor(w_t, dtype=torch.float64, requires_grad=True)
    S = q @ k.T
    R = torch.where(S >= 0, S, torch.zeros_like(S)) if ge else torch.where(S > 0, S, torch.zeros_like(S))
    I = w @ R
    p = torch.tensor(p_t, dtype=torch.float64)
    loss = torch.sum(p * (torch.log(p) - torch.log_softmax(I, dim=0)))
    loss.backward()
    return q.grad.numpy(), k.grad.numpy(), w.grad.numpy()


def test_kink_allowance_covers_the_other_decision(torch_cpu):
    torch = torch_cpu
    rng = np.random.default_rng(4)
    G, D, K = 3, 4, 5
    q_t = rng.normal(size=(G, D))
    k_sel = rng.normal(size=(K, D))
    # head 1 and slot 2 meet exactly at S = 0: q = (1, 1, 0, 0), k = (1, -1, 0, 0)
    q_t[1] = [1.0, 1.0, 0.0, 0.0]
    k_sel[2] = [1.0, -1.0, 0.0, 0.0]
    w_t = np.array([0.7, -1.3, 0.4])
    p_t = rng.dirichlet(np.ones(K))
    S = q_t @ k_sel.T
    assert S[1, 2] == 0.0
    off = np.abs(S) > 1e-2
    off[1, 2] = True
    assert off.all(), "only the planted pair may be near 0"
    valid = np.ones(K, dtype=bool)
    y, dq, dw, dk, dq_kink, dk_kink, scale = unit_backward(q_t, k_sel, valid, w_t, p_t, kink=True)
    gq0, gk0, gw0 = _unit_grads_torch(torch, q_t, k_sel, w_t, p_t, ge=False)
    gq1, gk1, gw1 = _unit_grads_torch(torch, q_t, k_sel, w_t, p_t, ge=True)
    # the oracle takes ReLU'(0) = 0 (reading 1) ...
    np.testing.assert_allclose(dq, gq0, atol=1e-13)
    np.testing.assert_allclose(dk, gk0, atol=1e-13)
    # ... and its allowance is exactly the change the other decision makes
    np.testing.assert_allclose(np.abs(gq1 - gq0), dq_kink, atol=1e-13)
    np.testing.assert_allclose(np.abs(gk1 - gk0), dk_kink, atol=1e-13)
    assert np.count_nonzero(dq_kink.any(axis=1)) == 1 and np.count_nonzero(dk_kink.any(axis=1)) == 1
    np.testing.assert_allclose(gw1, gw0, atol=1e-13)       # ReLU(0) = 0 either way
    # logit scale: max over slots of sum_h |w_h S_hs|
    assert scale == pytest.approx(float((np.abs(w_t) @ np.abs(S)).max()), rel=1e-15)


def test_kink_allowance_band_is_the_fp32_dot_product_bound():
    """Pairs with |S| just inside gamma_D sum|q k| count, just outside do not."""
    G, D, K = 1, 8, 2
    q_t = np.ones((G, D))
    k_sel = np.ones((K, D))
    bound = slikl_ref.gamma(D) * D                  # sum |q k| = D
    k_sel[0, 0] = 1.0 - D + 0.5 * bound              # S = 0.5 bound: inside
    k_sel[1, 0] = 1.0 - D + 2.0 * bound              # S = 2 bound: outside
    S = q_t @ k_sel.T
    mag = np.abs(q_t) @ np.abs(k_sel).T
    assert S[0, 0] <= slikl_ref.gamma(D) * mag[0, 0] < S[0, 1]
    out = unit_backward(q_t, k_sel, np.ones(K, dtype=bool), np.array([0.9]), np.array([0.3, 0.7]), kink=True)
    dq_kink, dk_kink = out[4], out[5]
    assert dk_kink[0].any() and not dk_kink[1].any()
    assert dq_kink.any()


def test_kink_outputs_leave_the_results_unchanged():
    x = _small(seed=11, n2=2, n1=6, duplicates=True)
    a = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, **_args(x))
    b = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, kink=True, **_args(x))
    for name in ("dq", "dk", "dw", "softmax_out"):
        assert np.array_equal(a[name], b[name])
    assert b["dq_kink"].shape == a["dq"].shape and b["dk_kink"].shape == a["dk"].shape
    assert b["logit_scale"].shape == a["softmax_out"].shape[:-1]
    # random data has no S within fp32 rounding of 0 at these sizes
    assert not b["dq_kink"].any() and not b["dk_kink"].any()
