"""GPU parity of the dense sibling operator (slikl_dense_grad, through the C ABI)
against its fp64 oracle (oracle/dense_ref.py), at the sparse operator's tolerances
(softmax_out max-abs 1e-5, dw max|err| / max|ref| 1e-3, dq / dk 1e-3 + 2e-2 |ref|
plus the kink allowance of the sparse oracle on the same visible keys)."""
import dataclasses
import sys

import numpy as np
import pytest

from oracle import dense_grad_ref, slikl_grad_ref, visible_keys
from tests.gpu_helpers import check_close
from workloads import DENSE_WORKLOADS, Workload, make_dense_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_token_amd as slikl
    slikl.load()


def W(**kw):
    base = dict(name="dense", layout="BSND", batch=1, s1=64, s2=64, n1=8, n2=1, d=32, topk=1,
                dtype="bf16", w_var=0.5, p_var=1.0, seed=41)
    base.update(kw)
    return Workload(**base)


CASES = {
    "m3_h64_d128_square": (W(batch=2, s1=150, s2=150, n1=64, d=128, w_var=1 / 8, p_var=2.0), 3),
    "m3_s1_lt_s2": (W(s1=70, s2=200, n1=32, d=128, w_var=1 / 8), 3),
    "m3_s1_gt_s2_f16": (W(s1=90, s2=40, n1=16, d=64, dtype="f16"), 3),
    "m0_h128_d64": (W(s1=40, s2=90, n1=128, d=64, w_var=1 / 16), 0),
    "m3_tnd_empty": (W(layout="TND", seqlens=(50, 0, 1, 120), n1=8, d=32), 3),
    "m0_tnd_n2_dirichlet": (W(layout="TND", seqlens=(60, 33), n1=64, n2=2, d=64, p_mode="dirichlet",
                              p_alpha=0.1, w_var=1 / 8), 0),
    "m3_len2048": (W(s1=48, s2=2048, n1=16, d=128, w_var=1 / 4), 3),
}


def _device(x):
    import torch
    tdt = torch.bfloat16 if x.wl.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    return dict(q=b16(x.q_bits), k=b16(x.k_bits), w=torch.from_numpy(np.ascontiguousarray(x.w)).cuda(),
                p=torch.from_numpy(np.ascontiguousarray(x.p)).cuda(),
                cu_q=None if x.cu_q is None else torch.from_numpy(x.cu_q.astype(np.int32)).cuda(),
                cu_k=None if x.cu_k is None else torch.from_numpy(x.cu_k.astype(np.int32)).cuda())


def _run(x, t, **kw):
    import torch
    import sparse_attention_indexer_token_amd as slikl
    mx = dict(max_seqlen_q=x.max_seqlen_q, max_seqlen_k=x.max_seqlen_k) if x.layout_q == "TND" else {}
    dq, dk, dw, y = slikl.slikl_dense_grad(t["q"], t["k"], t["w"], t["p"], mask_mode=x.mask_mode,
                                           layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=t["cu_q"],
                                           cu_seqlens_k=t["cu_k"], **mx, **kw)
    torch.cuda.synchronize()
    return dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dw=dw.cpu().numpy(),
                softmax_out=y.cpu().numpy())


def _ref(x, rows=None):
    """Dense oracle, plus the kink allowance from the sparse oracle on the visible keys
    (the two are pinned equal on such index lists)."""
    args = dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    ref = dense_grad_ref(x.q, x.k, x.w, x.p, mask_mode=x.mask_mode, rows=rows, **args)
    L = x.p.shape[-1]
    n2 = x.k.shape[-2]
    idx = np.full(x.p.reshape(-1, n2, L).shape, -1, dtype=np.int32)
    if x.layout_q == "BSND":
        tabs = [(b * x.q.shape[1], x.q.shape[1], x.k.shape[1]) for b in range(x.batch)]
    else:
        tabs = [(int(x.cu_q[b]), int(x.cu_q[b + 1] - x.cu_q[b]), int(x.cu_k[b + 1] - x.cu_k[b]))
                for b in range(x.batch)]
    for q0, s1b, s2b in tabs:
        for t in range(s1b):
            n = visible_keys(x.mask_mode, t, s1b, s2b)
            idx[q0 + t, :, :n] = np.arange(n)
    kink = slikl_grad_ref(x.q, x.k, x.w, idx.reshape(x.p.shape), x.p, rows=rows, kink=True, **args)
    ref["dq_kink"], ref["dk_kink"] = kink["dq_kink"], kink["dk_kink"]
    return ref


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dk_mode,det", [("auto", False), ("scatter", True), ("dense", False), ("sorted", True)])
def test_dense_parity(name, dk_mode, det):
    wl, mask = CASES[name]
    x = make_dense_inputs(wl, mask)
    t = _device(x)
    _say(f"[dense] {name} dk_mode={dk_mode} det={det}")
    got = _run(x, t, dk_mode=dk_mode, deterministic=det)
    msgs = check_close(got, _ref(x), label=f"dense {name} {dk_mode}")
    _say(f"[dense] {name}: " + " | ".join(msgs))
    # positions a row does not see hold exactly 0
    seen = _ref_visible(x)
    assert np.all(got["softmax_out"].reshape(seen.shape)[~seen] == 0)


def _ref_visible(x):
    L = x.p.shape[-1]
    n2 = x.k.shape[-2]
    seen = np.zeros(x.p.reshape(-1, n2, L).shape, dtype=bool)
    if x.layout_q == "BSND":
        tabs = [(b * x.q.shape[1], x.q.shape[1], x.k.shape[1]) for b in range(x.batch)]
    else:
        tabs = [(int(x.cu_q[b]), int(x.cu_q[b + 1] - x.cu_q[b]), int(x.cu_k[b + 1] - x.cu_k[b]))
                for b in range(x.batch)]
    for q0, s1b, s2b in tabs:
        for t in range(s1b):
            seen[q0 + t, :, :visible_keys(x.mask_mode, t, s1b, s2b)] = True
    return seen


def test_dense_metadata_and_determinism():
    """The dense pre-pass's metadata gives the same bits as the call's own, and
    deterministic mode is bitwise reproducible."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_dense_inputs(*CASES["m3_h64_d128_square"])
    t = _device(x)
    base = _run(x, t, deterministic=True)
    for mode, parts in (("weighted", 7), ("rows", 300)):
        md = slikl.slikl_dense_grad_metadata(t["q"], t["k"], t["p"], mask_mode=3, num_parts=parts, split_mode=mode,
                                             deterministic=True)
        got = _run(x, t, deterministic=True, metadata=md, num_parts=parts)
        for n in base:
            assert np.array_equal(base[n], got[n]), (mode, n)


def test_dense_rejects_what_it_does_not_build():
    import sparse_attention_indexer_token_amd as slikl
    x = make_dense_inputs(*CASES["m3_s1_lt_s2"])
    t = _device(x)
    with pytest.raises(slikl.SliklError) as e:
        slikl.slikl_dense_grad(t["q"], t["k"], t["w"], t["p"], mask_mode=3, cmp_ratio=4)
    assert e.value.status == 3            # compression: UNSUPPORTED
    with pytest.raises(slikl.SliklError) as e:
        slikl.slikl_dense_grad(t["q"], t["k"], t["w"], t["p"], mask_mode=1)
    assert e.value.status == 2            # mask mode outside {0, 3}: PARAM_INVALID


def test_dense_full_size():
    """The dense operator at the DeepSeek indexer's width over 2048-key rows (two
    sequences, rightDownCausal): every output against the oracle."""
    wl, mask = DENSE_WORKLOADS["dense_dsv32_2k"]
    x = make_dense_inputs(wl, mask)
    t = _device(x)
    _say(f"[dense full] T1={x.t1} visible={x.visible}")
    got = _run(x, t)
    from tests.oracle_pool import oracle_full
    # the dense problem as index lists of the visible keys, computed over row pieces
    L = x.p.shape[-1]
    idx = np.full(x.p.shape, -1, dtype=np.int32)
    for tt in range(x.q.shape[1]):
        n = visible_keys(mask, tt, x.q.shape[1], x.k.shape[1])
        idx[:, tt, :, :n] = np.arange(n)
    sx = dataclasses.replace(x)
    sx.idx = idx
    ref = oracle_full(sx, kl=False)
    flat = dict(dq=got["dq"].reshape(ref["dq"].shape), dk=got["dk"].reshape(ref["dk"].shape),
                dw=got["dw"].reshape(ref["dw"].shape), softmax_out=got["softmax_out"].reshape(ref["softmax_out"].shape))
    msgs = check_close(flat, ref, label="dense full")
    _say("[dense full] " + " | ".join(msgs))
    # the dense oracle itself on sampled rows (the two oracles are pinned equal)
    rows = np.array([0, 1, 777, 2047, 2048, 3000, 4095])
    dref = dense_grad_ref(x.q, x.k, x.w, x.p, mask_mode=mask, rows=rows)
    for n in ("dq", "dw", "softmax_out"):
        a = dref[n].reshape((x.t1,) + dref[n].shape[2:])[rows]
        b = ref[n][rows]
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
