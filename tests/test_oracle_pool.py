"""The row-piece runner of the full-size parity tests gives the oracle's results:
the same values as one whole-problem call (dk up to fp64 summation order)."""
import numpy as np
import pytest

from oracle import kl_per_unit_ref, slikl_grad_ref
from tests.oracle_pool import oracle_full
from workloads import Workload, make_inputs


def _wl(**kw):
    base = dict(name="pool", layout="BSND", batch=2, s1=37, s2=45, n1=8, n2=2, d=32, topk=24,
                dtype="bf16", w_var=0.5, index_mode="random", invalid_frac=0.2, duplicates=True,
                seed=3)
    base.update(kw)
    return Workload(**base)


@pytest.mark.parametrize("wl", [_wl(), _wl(layout="TND", seqlens=(30, 0, 41, 1), n2=1, dtype="f16"),
                                _wl(index_mode="sink_zipf", sink_keys=4, n2=1)],
                         ids=["bsnd_n2_dups", "tnd_empty", "sink_zipf"])
def test_pieces_equal_one_call(wl):
    x = make_inputs(wl)
    ref = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                         cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    kl = kl_per_unit_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                         cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    got = oracle_full(x, n_workers=3, pieces_per_worker=3)
    n1, d = x.q.shape[-2:]
    n2, topk = x.idx.shape[-2:]
    assert np.array_equal(got["dq"], ref["dq"].reshape(-1, n1, d))
    assert np.array_equal(got["dw"], ref["dw"].reshape(-1, n1))
    assert np.array_equal(got["softmax_out"], ref["softmax_out"].reshape(-1, n2, topk))
    assert np.array_equal(got["kl_loss"], kl)
    np.testing.assert_allclose(got["dk"], ref["dk"].reshape(-1, n2, d), rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.sort(got["rows"]), np.arange(x.t1))
    kref = slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                          cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, kink=True)
    assert np.array_equal(got["dq_kink"], kref["dq_kink"].reshape(-1, n1, d))
    np.testing.assert_allclose(got["dk_kink"], kref["dk_kink"].reshape(-1, n2, d), rtol=1e-12, atol=1e-12)
    assert np.array_equal(got["logit_scale"], kref["logit_scale"].reshape(-1, n2))
