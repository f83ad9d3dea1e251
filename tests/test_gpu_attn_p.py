"""GPU parity of the p producer (slikl_attn_softmax_l1norm, through the C ABI)
against the fp64 oracle oracle.attn_p_ref.

Tolerance, derived from the arithmetic: the kernel forms z = scale q . k with fp32
MFMA accumulation of exact 16-bit products over Dm terms, whose error is of order
sqrt(Dm) u sum_d |q_d k_d| (u = 2^-24); P = exp(z - lse) then carries that error
relative to P (the same for the log-sum-exp it computes), and p = a / sum(a) at most
twice it.  Per unit:  |p_gpu - p_ref| <= rho p_ref + 1e-10,
  rho = 4 scale sqrt(Dm) u max_{h,s} sum_d |q_hd k_sd| + 64 u
(the last term for the fp32 exp2 / log2 and the sums).  Rows must also sum to 1 and
be 0 at -1 slots; results are bitwise reproducible.
"""
import dataclasses
import sys

import numpy as np
import pytest

from oracle import attn_softmax_l1norm_ref, lse_over_slots_ref
from workloads import ATTN_P_WORKLOADS, AttnPWorkload, Workload, make_attn_p_inputs

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


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


def IW(**kw):
    base = dict(name="pidx", layout="BSND", batch=1, s1=64, s2=64, n1=8, n2=1, d=32, topk=16,
                dtype="bf16", w_var=0.5, index_mode="causal", p_var=1.0, seed=31)
    base.update(kw)
    return Workload(**base)


CASES = {
    "h128_d576": AttnPWorkload(name="a", index=IW(batch=2, s1=70, s2=90, topk=128), nm=128, dm=576, seed=1),
    "h64_d128_f16_dups": AttnPWorkload(name="b", index=IW(s1=100, s2=120, topk=200, dtype="f16", index_mode="random",
                                                          invalid_frac=0.3, duplicates=True), nm=64, dm=128,
                                       scale=0.09, seed=2),
    "h16_d64_tnd": AttnPWorkload(name="c", index=IW(layout="TND", seqlens=(50, 0, 1, 77), topk=40), nm=16, dm=64,
                                 scale=0.125, seed=3),
    "h32x2_d256_n2": AttnPWorkload(name="d", index=IW(batch=2, s1=40, s2=60, n1=64, n2=2, topk=96), nm=64, dm=256,
                                   scale=0.0625, seed=4),
    "h100_d512_ragged": AttnPWorkload(name="e", index=IW(s1=33, s2=45, topk=300, index_mode="random",
                                                         invalid_frac=0.5), nm=100, dm=512, scale=0.04, seed=5),
    "topk1": AttnPWorkload(name="f", index=IW(s1=20, s2=20, topk=1), nm=32, dm=128, seed=6),
    "no_valid_rows": AttnPWorkload(name="g", index=IW(s1=16, s2=16, topk=24, index_mode="random", invalid_frac=1.0),
                                   nm=8, dm=64, seed=7),
    "full_topk2048": AttnPWorkload(name="h", index=IW(s1=40, s2=2100, topk=2048, index_mode="random",
                                                      invalid_frac=0.1), nm=48, dm=576, seed=8),
}


def _device(x):
    import torch
    tdt = torch.bfloat16 if x.wl.index.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

    return dict(q=b16(x.qm_bits), k=b16(x.km_bits), idx=torch.from_numpy(np.ascontiguousarray(x.idx)).cuda(),
                cu_q=None if x.cu_q is None else torch.from_numpy(x.cu_q.astype(np.int32)).cuda(),
                cu_k=None if x.cu_k is None else torch.from_numpy(x.cu_k.astype(np.int32)).cuda())


def _run(x, t, lse=None):
    import torch
    import sparse_attention_indexer_token_amd as slikl
    lt = None if lse is None else torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda()
    out = torch.full(t["idx"].shape, float("nan"), dtype=torch.float32, device="cuda")
    slikl.slikl_attn_softmax_l1norm(t["q"], t["k"], t["idx"], x.wl.scale, lse=lt, out=out, layout_q=x.layout_q,
                                    layout_k=x.layout_k, cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _rho(x):
    nm, dm = x.qm.shape[-2:]
    n2 = x.km.shape[-2]
    qa = np.abs(x.qm.reshape(-1, nm, dm)).max(axis=(0, 1))
    ka = np.abs(x.km.reshape(-1, n2, dm)).max(axis=(0, 1))
    bound = float(qa @ ka)                    # >= max_{h,s} sum_d |q_hd k_sd|
    return 4 * x.wl.scale * np.sqrt(dm) * U32 * bound + 64 * U32


def _check(got, ref, x, label):
    valid = x.idx >= 0
    assert np.all(np.isfinite(got)), label
    assert np.all(got[~valid] == 0), label
    rho = _rho(x)
    err = np.abs(got.astype(np.float64) - ref.reshape(got.shape))
    bound = rho * np.abs(ref.reshape(got.shape)) + 1e-10
    worst = float((err / bound).max()) if err.size else 0.0
    _say(f"[attn_p] {label}: rho {rho:.2e}, max rel err {float((err / np.maximum(ref.reshape(got.shape), 1e-30))[valid].max()) if valid.any() else 0:.2e}, worst err/bound {worst:.3f}")
    assert np.all(err <= bound), label
    sums = got.sum(-1)[valid.any(-1)]
    assert np.all(np.abs(sums - 1) < 1e-5), label


def _ref(x, lse=None):
    return attn_softmax_l1norm_ref(x.qm, x.km, x.idx, scale=x.wl.scale, lse=lse, layout_q=x.layout_q,
                                   layout_k=x.layout_k, cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)


@pytest.mark.parametrize("name", list(CASES))
def test_attn_p_parity(name):
    x = make_attn_p_inputs(CASES[name])
    t = _device(x)
    _say(f"[attn_p] {name}")
    got = _run(x, t)
    _check(got, _ref(x), x, name)
    again = _run(x, t)
    assert np.array_equal(got, again), "bitwise reproducible"


@pytest.mark.parametrize("name", ["h128_d576", "h64_d128_f16_dups", "h16_d64_tnd"])
def test_attn_p_with_given_lse(name):
    """lse given: over the slots (equal to the computed one) and over a larger,
    dense key set (every key of the batch), where the L1 normalisation matters."""
    x = make_attn_p_inputs(CASES[name])
    t = _device(x)
    lse_s = lse_over_slots_ref(x.qm, x.km, x.idx, scale=x.wl.scale, layout_q=x.layout_q, layout_k=x.layout_k,
                               cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    lse_s = np.where(np.isfinite(lse_s), lse_s, 0.0)
    _check(_run(x, t, lse=lse_s), _ref(x, lse=lse_s), x, f"{name} slot lse")
    # dense lse: over every key of the row's batch (the oracle's fp64, from the inputs)
    from tests.oracle_pool import batch_tables
    nm, dm = x.qm.shape[-2:]
    n2 = x.km.shape[-2]
    qf = x.qm.reshape(-1, nm, dm).astype(np.float64)
    kf = x.km.reshape(-1, n2, dm).astype(np.float64)
    qt, kt = batch_tables(x)
    lse_d = np.zeros((qf.shape[0], nm))
    hm = nm // n2
    for (q0, nq), (k0, nk) in zip(qt, kt):
        for g in range(n2):
            if nk == 0 or nq == 0:
                continue
            z = x.wl.scale * np.einsum("rhd,kd->rhk", qf[q0:q0 + nq, g * hm:(g + 1) * hm], kf[k0:k0 + nk, g])
            top = z.max(-1, keepdims=True)
            lse_d[q0:q0 + nq, g * hm:(g + 1) * hm] = top[..., 0] + np.log(np.exp(z - top).sum(-1))
    lse_d = lse_d.reshape(x.qm.shape[:-1])
    _check(_run(x, t, lse=lse_d), _ref(x, lse=lse_d), x, f"{name} dense lse")


def test_attn_p_out_of_range_indices_are_skipped():
    x = make_attn_p_inputs(CASES["h64_d128_f16_dups"])
    x.idx[0, 5, 0, 3] = 10_000
    x.idx[0, 9, 0, 4] = -9
    t = _device(x)
    got = _run(x, t)
    x.idx[0, 5, 0, 3] = -1
    x.idx[0, 9, 0, 4] = -1
    _check(got, _ref(x), x, "out of range skipped")


def test_attn_p_full_size():
    """The DeepSeek-shaped main attention (128 heads, Dm 576) over the indexer's causal
    top-2048 lists: every row against the whole-problem oracle."""
    from tests.oracle_pool import attn_p_full
    x = make_attn_p_inputs(ATTN_P_WORKLOADS["attn_p_dsv32"])
    t = _device(x)
    _say(f"[attn_p full] running T1={x.t1} valid={x.valid_slots}")
    got = _run(x, t)
    _say("[attn_p full] oracle")
    ref = attn_p_full(x)
    _check(got, ref, x, "attn_p_dsv32")
