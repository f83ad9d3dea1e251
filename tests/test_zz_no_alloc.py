"""The entry point that allocates nothing (slikl_grad_noalloc): its outputs equal
those of slikl_grad with a caller workspace, on two calls in a row, the second
with a smaller input (the fixed array keeps the first call's contents)."""
import sys

import numpy as np
import pytest

from tests.gpu_helpers import check_close, oracle, run_gpu, to_device
from workloads import WORKLOADS, Workload, make_inputs

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


def _wl(**kw):
    base = dict(name="noalloc", layout="BSND", batch=2, s1=300, s2=320, n1=64, n2=1, d=128, topk=256,
                dtype="bf16", w_var=1 / 8, index_mode="causal", p_var=2.0, seed=21)
    base.update(kw)
    return Workload(**base)


def _noalloc(x, t, **kw):
    import torch
    import sparse_attention_indexer_token_amd as slikl
    out = (torch.full_like(t["q"], 7), torch.full_like(t["k"], 7), torch.full_like(t["w"], 7),
           torch.full_like(t["p"], 7))
    slikl.slikl_grad_noalloc(t["q"], t["k"], t["w"], t["idx"], t["p"], out=out, layout_q=x.layout_q,
                             layout_k=x.layout_k, cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"], **kw)
    torch.cuda.synchronize()
    dq, dk, dw, y = out
    return dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dw=dw.cpu().numpy(),
                softmax_out=y.cpu().numpy())


def _strategy(x, t, **kw):
    import sparse_attention_indexer_token_amd as slikl
    desc = slikl.make_desc(t["q"], t["k"], t["idx"], layout_q=x.layout_q, layout_k=x.layout_k,
                           cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"], **kw)
    return slikl.slikl_grad_noalloc_strategy(desc)


# (first input, second smaller input, call options); the strategy the fixed array allows
CASES = [
    ("auto_dense", _wl(), _wl(batch=1, s1=150, s2=170, seed=22), dict(deterministic=False)),
    ("det_scatter", _wl(index_mode="sink_zipf", invalid_frac=0.1, sink_keys=8, n1=16, topk=64),
     _wl(index_mode="sink_zipf", invalid_frac=0.1, sink_keys=8, n1=16, topk=64, batch=1, s1=90, s2=90,
         seed=23), dict(deterministic=True, dk_mode="scatter")),
    ("sorted_tnd", _wl(layout="TND", seqlens=(200, 0, 130), dtype="f16"),
     _wl(layout="TND", seqlens=(60, 41), dtype="f16", seed=24), dict(deterministic=True, dk_mode="sorted")),
]


@pytest.mark.parametrize("name,first,second,opts", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_slikl_grad(name, first, second, opts):
    for i, wl in enumerate((first, second)):
        x = make_inputs(wl)
        t = to_device(x)
        mx = dict(max_seqlen_q=x.max_seqlen_q, max_seqlen_k=x.max_seqlen_k) if x.layout_q == "TND" else {}
        strat = _strategy(x, t, **opts, **mx)
        _say(f"[noalloc] {name} call {i + 1}: T1={x.t1} strategy={strat}")
        got = _noalloc(x, t, **opts, **mx)
        base = run_gpu(x, t, dk_mode=strat, deterministic=opts.get("deterministic", False))
        for n in ("dq", "dw", "softmax_out"):
            assert np.array_equal(got[n], base[n]), (name, i, n)
        if opts.get("deterministic", False) or strat == "dense":
            assert np.array_equal(got["dk"], base["dk"]), (name, i, "dk")
        check_close(got, oracle(x), label=f"noalloc {name} call {i + 1}")


def test_noalloc_full_size_falls_back_to_scatter():
    """The DeepSeek-shaped workload: AUTO's dense records do not fit the fixed array,
    so the call runs the scatter strategy (fp32 atomics: dk equal up to summation
    order); a second, smaller call follows."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(WORKLOADS["dsv32_indexer"])
    t = to_device(x)
    assert _strategy(x, t) == "scatter"
    _say("[noalloc] dsv32_indexer full size")
    got = _noalloc(x, t)
    base = run_gpu(x, t, dk_mode="scatter")
    for n in ("dq", "dw", "softmax_out"):
        assert np.array_equal(got[n], base[n]), n
    check_close({"dk": got["dk"]}, {"dk": base["dk"]}, what=("dk",), label="noalloc dsv32 dk vs slikl_grad")
    x2 = make_inputs(_wl(batch=1, s1=64, s2=64, topk=48, seed=25))
    t2 = to_device(x2)
    got2 = _noalloc(x2, t2)
    check_close(got2, oracle(x2), label="noalloc second call")
    # an explicit strategy whose workspace exceeds the array is refused, nothing launched
    with pytest.raises(slikl.SliklError) as err:
        slikl.slikl_grad_noalloc(t["q"], t["k"], t["w"], t["idx"], t["p"], dk_mode="dense",
                                 out=(torch.empty_like(t["q"]), torch.empty_like(t["k"]),
                                      torch.empty_like(t["w"]), torch.empty_like(t["p"])))
    assert err.value.status == 4
