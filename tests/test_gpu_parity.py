"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases are compared element by element on every output; they span
several chunks, ragged tails, every head-tile width (32/64/128 padded heads),
D in {32, 64, 128}, fp16 and bf16, N2 = 2, TND with an empty sequence,
duplicates, interleaved -1, rows without any valid slot and topk = 1.
The five headline workloads run at full size in the benchmark's launch
configuration; there every row and every key is compared with the whole-problem
oracle (computed over row pieces in worker processes, tests/oracle_pool.py).
"""
import sys

import numpy as np
import pytest

from workloads import WORKLOADS, Workload, make_inputs
from tests.gpu_helpers import check_close, max_seqlens, oracle, run_gpu, to_device

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
    slikl.load()          # fail loudly when the library is missing


def W(**kw):
    base = dict(name="case", layout="BSND", batch=1, s1=64, s2=64, n1=8, n2=1, d=32, topk=16,
                dtype="bf16", w_var=0.5, index_mode="causal", p_var=1.0, seed=7)
    base.update(kw)
    return Workload(**base)


SMALL = {
    "tiny_causal": WORKLOADS["tiny_causal"],
    "hp64_d128_ragged": W(batch=2, s1=150, s2=170, n1=64, d=128, topk=200, w_var=1 / 8, p_var=2.0),
    "hp32_d128_f16_dups": W(s1=120, s2=130, n1=32, d=128, topk=300, dtype="f16", w_var=1 / 8,
                            index_mode="random", invalid_frac=0.3, duplicates=True),
    "hp128_d64": W(s1=70, s2=90, n1=128, d=64, topk=100, w_var=1 / 16, index_mode="random",
                   invalid_frac=0.1),
    "hp64_d64_n2": W(batch=2, s1=40, s2=60, n1=128, n2=2, d=64, topk=96, w_var=1 / 8),
    "g8_d32_tnd": W(layout="TND", seqlens=(50, 1, 0, 90), n1=8, d=32, topk=40),
    "f16_dirichlet_tnd": W(layout="TND", seqlens=(130, 70), n1=64, d=128, topk=128, dtype="f16",
                           w_var=1 / 8, p_mode="dirichlet", p_alpha=0.1),
    "topk1": W(s1=50, s2=50, n1=16, d=64, topk=1),
    "no_valid_rows": W(s1=30, s2=30, n1=32, d=32, topk=24, index_mode="random", invalid_frac=1.0),
    "sink_zipf_small": W(batch=2, s1=200, s2=200, n1=16, d=128, topk=64, index_mode="sink_zipf",
                         invalid_frac=0.1, sink_keys=8, w_var=0.25),
    "g1_d128": W(s1=40, s2=40, n1=1, d=128, topk=33),
    "g100_d32": W(s1=20, s2=50, n1=100, d=32, topk=70, w_var=1 / 16),
}


DK_MODES = [("scatter", False), ("scatter", True), ("dense", False), ("sorted", False), ("sorted", True)]



@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("dk_mode,det", DK_MODES)
def test_small_parity(name, dk_mode, det):
    x = make_inputs(SMALL[name])
    _say(f"[parity] {name} dk_mode={dk_mode} det={det}")
    got = run_gpu(x, deterministic=det, dk_mode=dk_mode)
    ref = oracle(x)
    check_close(got, ref, label=name)
    if name == "no_valid_rows":
        assert np.all(got["dq"] == 0) and np.all(got["dk"] == 0) and np.all(got["softmax_out"] == 0)


# KL output tolerance per unit: |got - ref| <= 1e-4 (1 + |ref|).  The unit's value
# moves by sum_s (p_s - y_s) dI_s under errors dI in I, i.e. by at most 2 max |dI|;
# I comes from fp32-accumulated 16-bit products (relative error ~ D 2^-24 per S,
# ~1e-5 of |I| at D = 128), and the fp32 logs and the 2048-term fp32 sum add ~1e-5 of
# the value.
@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("dk_mode", ["scatter", "dense", "sorted"])
def test_kl_loss_output(name, dk_mode):
    from oracle import kl_per_unit_ref
    x = make_inputs(SMALL[name])
    _say(f"[kl] {name} dk_mode={dk_mode}")
    got = run_gpu(x, kl=True, dk_mode=dk_mode)
    ref = kl_per_unit_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                          cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    g = got["kl_loss"].reshape(ref.shape).astype(np.float64)
    assert np.all(np.isfinite(g))
    excess = np.abs(g - ref) - 1e-4 * (1 + np.abs(ref))
    assert np.max(excess) <= 0, (name, float(np.max(excess)))
    # the other outputs are unchanged by asking for the loss
    check_close(got, oracle(x), label=f"{name} with kl")


def test_metadata_matches_reference():
    """Integer metadata: bit-exact against the reference split, both modes."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    from oracle.metadata_ref import metadata_ref
    for name in ("hp64_d128_ragged", "g8_d32_tnd", "sink_zipf_small"):
        x = make_inputs(SMALL[name])
        t = to_device(x)
        for mode, parts in (("weighted", 37), ("rows", 37), ("weighted", 1), ("rows", 2048)):
            _say(f"[metadata] {name} {mode} {parts}")
            md = slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], layout_q=x.layout_q,
                                           layout_k=x.layout_k, cu_seqlens_q=t["cu_q"],
                                           cu_seqlens_k=t["cu_k"], num_parts=parts, split_mode=mode)
            torch.cuda.synchronize()
            desc = slikl.make_desc(t["q"], t["k"], t["idx"], layout_q=x.layout_q, layout_k=x.layout_k,
                                   cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"], num_parts=parts,
                                   split_mode=mode)
            want = metadata_ref(layout_q=x.layout_q, layout_k=x.layout_k, batch=x.batch,
                                s1=x.s1, s2=x.s2, n2=x.wl.n2, topk=x.wl.topk, parts=parts,
                                mode=0 if mode == "weighted" else 1,
                                overhead=slikl.slikl_grad_unit_overhead(desc),
                                cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k,
                                sparse_indices=x.idx.reshape(-1, x.wl.n2, x.wl.topk))
            assert np.array_equal(md.cpu().numpy(), want)


def test_results_do_not_depend_on_metadata():
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(SMALL["hp64_d128_ragged"])
    t = to_device(x)
    base = run_gpu(x, t)
    base_det = run_gpu(x, t, deterministic=True)
    for mode, parts in (("rows", 3), ("weighted", 5), ("rows", 2048), ("weighted", 1)):
        _say(f"[metadata-independence] {mode} {parts}")
        md = slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], num_parts=parts, split_mode=mode)
        got = run_gpu(x, t, metadata=md, num_parts=parts)
        for name in ("dq", "dw", "softmax_out"):
            assert np.array_equal(got[name], base[name]), name
        check_close(got, oracle(x), what=("dk",))
        got_det = run_gpu(x, t, deterministic=True, metadata=md, num_parts=parts)
        for name in ("dq", "dk", "dw", "softmax_out"):
            assert np.array_equal(got_det[name], base_det[name]), name
    torch.cuda.synchronize()


@pytest.mark.parametrize("dk_mode", ["scatter", "dense", "sorted"])
def test_deterministic_mode_is_bitwise_reproducible(dk_mode):
    import torch
    x = make_inputs(SMALL["sink_zipf_small"])
    t = to_device(x)
    first = run_gpu(x, t, deterministic=True, dk_mode=dk_mode)
    s = torch.cuda.Stream()
    for i in range(9):
        if i % 2:
            with torch.cuda.stream(s):
                again = run_gpu(x, t, deterministic=True, dk_mode=dk_mode)
        else:
            again = run_gpu(x, t, deterministic=True, dk_mode=dk_mode)
        for name in first:
            assert np.array_equal(first[name], again[name]), (i, name)
    check_close(first, run_gpu(x, t, deterministic=False, dk_mode="scatter"), what=("dk",))


@pytest.mark.parametrize("dk_mode", ["scatter", "dense", "sorted"])
def test_slot_order_and_padding_invariance(dk_mode):
    """Permuting the slots (with -1 padding interleaved) permutes softmax_out and
    leaves dq, dk, dw within tolerance (the fp16 rounding of dS may move by an
    ulp with the summation order, so equality is not expected)."""
    x = make_inputs(SMALL["hp64_d128_ragged"])
    a = run_gpu(x, dk_mode=dk_mode)
    perm = np.random.default_rng(5).permutation(x.idx.shape[-1])
    x2 = make_inputs(SMALL["hp64_d128_ragged"])
    x2.idx = np.ascontiguousarray(x2.idx[..., perm])
    x2.p = np.ascontiguousarray(x2.p[..., perm])
    b = run_gpu(x2, dk_mode=dk_mode)
    check_close(b, dict(a, softmax_out=a["softmax_out"][..., perm]), what=("softmax_out",))
    check_close(b, oracle(x2), label="permuted slots")


def test_out_of_range_index_is_skipped_and_flagged():
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(SMALL["hp64_d128_ragged"])
    x.idx[0, 5, 0, 0] = 10_000           # outside [0, S2)
    x.idx[1, 7, 0, 1] = -7               # negative, not -1
    t = to_device(x)
    got = run_gpu(x, t)
    md = slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], num_parts=8)
    torch.cuda.synchronize()
    assert md[8].item() & 4
    x.idx[0, 5, 0, 0] = -1
    x.idx[1, 7, 0, 1] = -1
    check_close(got, oracle(x), label="out-of-range skipped")


def test_tnd_sequence_longer_than_its_given_maximum_is_flagged():
    """Dense strategy with TND sides given a maximum below the longest sequence: the
    call completes, keys past the maximum act as -1 slots (dq, dw and softmax_out then
    match the oracle on those indices), and the metadata error word has bit 8."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(SMALL["g8_d32_tnd"])          # sequences of 50, 1, 0 and 90 rows
    t = to_device(x)
    lim = 60
    _say("[tnd max] g8_d32_tnd, maxima 60 < 90")
    kw = dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"],
              dk_mode="dense", max_seqlen_q=lim, max_seqlen_k=lim)
    md = slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], **kw)
    dq, dk, dw, y = slikl.slikl_grad(t["q"], t["k"], t["w"], t["idx"], t["p"], metadata=md, **kw)
    torch.cuda.synchronize()
    assert int(md[8].item()) & 8
    idx2 = np.where(x.idx >= lim, -1, x.idx)
    from oracle import slikl_grad_ref
    ref = slikl_grad_ref(x.q, x.k, x.w, idx2, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                         cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k)
    got = dict(dq=dq.float().cpu().numpy(), dw=dw.cpu().numpy(), softmax_out=y.cpu().numpy())
    check_close(got, ref, what=("dq", "dw", "softmax_out"), label="tnd max")
    # rows past the given maximum add nothing to dk
    row_b = np.searchsorted(x.cu_q, np.arange(x.t1), side="right") - 1
    kept = np.flatnonzero(np.arange(x.t1) - x.cu_q[row_b] < lim)
    ref_k = slikl_grad_ref(x.q, x.k, x.w, idx2, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                           cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=kept)
    check_close(dict(dk=dk.float().cpu().numpy()), ref_k, what=("dk",), label="tnd max dk")
    # within the maxima nothing is flagged
    md_ok = slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], **dict(kw, **max_seqlens(x)))
    torch.cuda.synchronize()
    assert int(md_ok[8].item()) & 8 == 0


@pytest.mark.parametrize("dk_mode", ["scatter", "dense", "sorted"])
def test_profiled_call_matches_and_times_phases(dk_mode):
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(SMALL["hp64_d128_ragged"])
    t = to_device(x)
    base = run_gpu(x, t, dk_mode=dk_mode, deterministic=True)
    (dq, dk, dw, y), ms = slikl.slikl_grad_profiled(t["q"], t["k"], t["w"], t["idx"], t["p"],
                                                    dk_mode=dk_mode, deterministic=True)
    torch.cuda.synchronize()
    got = dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dw=dw.cpu().numpy(),
               softmax_out=y.cpu().numpy())
    for name in got:
        assert np.array_equal(got[name], base[name]), name
    assert ms["fused"] > 0 and ms["dk_final"] > 0 and ms["metadata"] > 0
    # a separate dK phase runs in the dense (key-major kernel) and sorted (slot parts
    # sorted by key, then summed per key) strategies; scatter adds dK inside the fused kernel
    assert (ms["dk"] > 0) == (dk_mode != "scatter")
    assert (ms["dk_prep"] > 0) == (dk_mode != "scatter")
    assert (ms["dk_reduce"] > 0) == (dk_mode == "sorted")


# Full-size cases, grouped by workload so that one oracle result serves them: the
# library's dK strategy, then strategies the default launch does not take at that
# size (fp32 atomics on the long context, the key-sorted sums on the DeepSeek shape
# and under the sink keys' contention).
FULL_CASES = [("tiny_causal", "auto"), ("dsv32_indexer", "auto"), ("dsv32_indexer", "sorted"),
              ("long_context", "auto"), ("long_context", "scatter"),
              ("contention_det", "auto"), ("contention_det", "sorted"), ("varlen_tnd", "auto")]
_FULL_REF = {}


def _full_ref(name):
    """Inputs and the whole-problem oracle of a headline workload (one kept at a time)."""
    if name not in _FULL_REF:
        _FULL_REF.clear()
        from tests.oracle_pool import oracle_full
        _say(f"[full] generating {name}")
        x = make_inputs(WORKLOADS[name])
        _say(f"[full] oracle over all {x.t1} rows of {name}")
        _FULL_REF[name] = (x, oracle_full(x))
    return _FULL_REF[name]


def _flat(got, x):
    n1, d = x.q.shape[-2:]
    n2, topk = x.idx.shape[-2:]
    out = dict(dq=got["dq"].reshape(-1, n1, d), dk=got["dk"].reshape(-1, n2, d),
               dw=got["dw"].reshape(-1, n1), softmax_out=got["softmax_out"].reshape(-1, n2, topk))
    if "kl_loss" in got:
        out["kl_loss"] = got["kl_loss"].reshape(-1, n2)
    return out


@pytest.mark.parametrize("name,dk_mode", FULL_CASES)
def test_full_size_every_output(name, dk_mode):
    """Headline workloads at full size in the benchmark's launch configuration
    (weighted metadata): every row of dq, dw, softmax_out and the loss terms, and
    every key of dk (the sink keys and the most referenced early keys included),
    against the whole-problem fp64 oracle."""
    x, ref = _full_ref(name)
    _say(f"[full] running {name} T1={x.t1} valid={x.valid_slots} dk_mode={dk_mode}")
    got = _flat(run_gpu(x, dk_mode=dk_mode, kl=True), x)
    msgs = check_close(got, ref, label=f"{name} {dk_mode}")
    _say(f"[full] {name} {dk_mode}: " + " | ".join(msgs))
    # the keys that most rows name (the scatter-add's hottest targets) reported apart
    n2, d = x.k.shape[-2:]
    flat = x.idx.reshape(-1, n2, x.idx.shape[-1])
    qt, kt = __import__("tests.oracle_pool", fromlist=["batch_tables"]).batch_tables(x)
    counts = np.zeros(x.t2, dtype=np.int64)
    for b, ((q0, nq), (k0, _)) in enumerate(zip(qt, kt)):
        ids = flat[q0:q0 + nq]
        counts += np.bincount((ids[ids >= 0] + k0).ravel(), minlength=x.t2)[:x.t2]
    hot = np.argsort(counts)[-64:]
    err = np.abs(got["dk"][hot].astype(np.float64) - ref["dk"][hot])
    bound = 1e-3 + 2e-2 * np.abs(ref["dk"][hot])
    _say(f"[full] {name} {dk_mode}: 64 hottest keys (named {counts[hot].min()}..{counts[hot].max()} "
         f"times), worst err/bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)
    kg = got["kl_loss"].astype(np.float64)
    assert np.all(np.isfinite(kg))
    assert np.max(np.abs(kg - ref["kl_loss"]) - 1e-4 * (1 + np.abs(ref["kl_loss"]))) <= 0, f"{name} kl_loss"
    # global invariants
    y = got["softmax_out"]
    valid = flat >= 0
    assert np.all(y[~valid] == 0)
    sums = y.sum(-1)[valid.any(-1)]
    assert np.max(np.abs(sums - 1)) < 1e-4


@pytest.mark.parametrize("dk_mode", ["auto", "sorted"])
def test_full_size_deterministic_is_bitwise_reproducible(dk_mode):
    """The contention workload at full size in deterministic mode: three runs with the
    weighted split and one with the even row split give identical bits in every
    output (the dense strategy's task table and the sorted strategy's multi-wave bins
    at their full sizes)."""
    x = make_inputs(WORKLOADS["contention_det"])
    t = to_device(x)
    _say(f"[full det] contention_det dk_mode={dk_mode}")
    first = run_gpu(x, t, deterministic=True, dk_mode=dk_mode)
    for i, split in enumerate(("weighted", "weighted", "rows")):
        again = run_gpu(x, t, deterministic=True, dk_mode=dk_mode, split_mode=split)
        for name in first:
            assert np.array_equal(first[name], again[name]), (i, split, name)


# Inputs at other scales: q, k ~ N(0, 16) (|S| near 180, peaky softmax rows), and a
# few key rows 100 times the rest (the fp16 copy of bf16 keys takes one global
# power-of-two scale from the largest key; fp16 keys must stay in range).
SCALES = {
    "bf16_var16": W(batch=2, s1=160, s2=200, n1=64, d=128, topk=192, q_var=16.0, k_var=16.0,
                    w_var=1 / 8, p_var=2.0),
    "f16_var16": W(batch=2, s1=160, s2=200, n1=64, d=128, topk=192, q_var=16.0, k_var=16.0,
                   w_var=1 / 8, p_var=2.0, dtype="f16"),
    "bf16_outlier_keys": W(batch=2, s1=160, s2=200, n1=64, d=128, topk=192, w_var=1 / 8, p_var=2.0,
                           k_outliers=6, k_outlier_scale=100.0),
    "f16_outlier_keys": W(batch=2, s1=160, s2=200, n1=32, d=128, topk=192, w_var=1 / 8, p_var=2.0,
                          k_outliers=6, k_outlier_scale=100.0, dtype="f16"),
}


@pytest.mark.parametrize("name", list(SCALES))
@pytest.mark.parametrize("dk_mode,det", [("scatter", False), ("dense", False), ("sorted", True)])
def test_input_scale(name, dk_mode, det):
    x = make_inputs(SCALES[name])
    _say(f"[scale] {name} dk_mode={dk_mode} det={det}")
    got = run_gpu(x, deterministic=det, dk_mode=dk_mode)
    # softmax_out: logits about ten times the pages' workloads' carry fp32 errors in
    # proportion; the bound scales with the unit's logit magnitude (check_close)
    msgs = check_close(got, oracle(x), label=name, y_logit_scaled=True)
    _say(f"[scale] {name}: " + " | ".join(msgs))


def test_seq_used_k_inside_a_key_block_with_stale_workspace():
    """Dense strategy, TND, seqUsedK cutting a batch's keys inside a dK key block that
    a used row's named range reaches; the workspace starts full of non-zero bytes, so
    any key read past the used length would show in dk."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    from oracle import slikl_grad_ref
    x = make_inputs(W(layout="TND", seqlens=(300, 200), n1=64, d=128, topk=256, w_var=1 / 8, p_var=2.0))
    used_q = np.array([300, 200], dtype=np.int32)
    used_k = np.array([250, 130], dtype=np.int32)
    row_b = np.searchsorted(x.cu_q, np.arange(x.t1), side="right") - 1
    idx = np.where(x.idx >= used_k[row_b][:, None, None], -1, x.idx).astype(np.int32)
    t = to_device(x)
    ti = torch.from_numpy(idx).cuda()
    kw = dict(layout_q="TND", layout_k="TND", cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"],
              seq_used_q=torch.from_numpy(used_q).cuda(), seq_used_k=torch.from_numpy(used_k).cuda(),
              **max_seqlens(x))
    ref = slikl_grad_ref(x.q, x.k, x.w, idx, x.p, layout_q="TND", layout_k="TND", cu_seqlens_q=x.cu_q,
                         cu_seqlens_k=x.cu_k, seq_used_q=used_q, seq_used_k=used_k)
    for dk_mode, det in (("dense", False), ("dense", True), ("sorted", False), ("scatter", True)):
        _say(f"[seq_used_k block] dk_mode={dk_mode} det={det}")
        desc = slikl.make_desc(t["q"], t["k"], ti, dk_mode=dk_mode, deterministic=det, **kw)
        ws = torch.full((slikl.slikl_grad_workspace_size(desc),), 0x3F, dtype=torch.uint8, device="cuda")
        dq, dk, dw, y = slikl.slikl_grad(t["q"], t["k"], t["w"], ti, t["p"], dk_mode=dk_mode,
                                         deterministic=det, workspace=ws, **kw)
        torch.cuda.synchronize()
        got = dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dw=dw.cpu().numpy(),
                   softmax_out=y.cpu().numpy())
        check_close(got, ref, label=f"seq_used_k block {dk_mode}")
        kb = x.cu_k[:-1]
        for b in range(2):
            assert np.all(got["dk"][kb[b] + used_k[b]:x.cu_k[b + 1]] == 0)


@pytest.mark.parametrize("dk_mode", ["scatter", "dense", "sorted"])
@pytest.mark.parametrize("name", ["g8_d32_tnd", "f16_dirichlet_tnd"])
def test_seq_used_lengths(name, dk_mode):
    """seqUsedQ / seqUsedK on TND inputs: rows past a batch's used length take no part
    (their indices are not flagged), indices past the used keys are skipped and flagged."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    from oracle import kl_per_unit_ref, slikl_grad_ref
    x = make_inputs(SMALL[name])
    nb = len(x.cu_q) - 1
    lens = np.diff(x.cu_q)
    used_q = np.array([(l * 2) // 3 if b % 2 == 0 else l for b, l in enumerate(lens)], dtype=np.int32)
    used_k = np.array([l if b % 2 == 0 else l // 2 for b, l in enumerate(lens)], dtype=np.int32)
    if nb > 1:
        used_q[-1] = 0                                   # a batch that takes no part
    t = to_device(x)
    uq = torch.from_numpy(used_q).cuda()
    uk = torch.from_numpy(used_k).cuda()
    kw = dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"],
              seq_used_q=uq, seq_used_k=uk)
    cleaned = x.idx.copy()
    row_b = np.searchsorted(x.cu_q, np.arange(x.t1), side="right") - 1
    row_in = np.arange(x.t1) - x.cu_q[row_b]
    for r in range(x.t1):
        cleaned[r] = np.where(cleaned[r] >= used_k[row_b[r]], -1, cleaned[r])
    ref = slikl_grad_ref(x.q, x.k, x.w, cleaned, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                         cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, seq_used_q=used_q, seq_used_k=used_k)
    kref = kl_per_unit_ref(x.q, x.k, x.w, cleaned, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                           cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, seq_used_q=used_q, seq_used_k=used_k)
    for variant in ("past_used_keys", "garbage_in_unused_rows"):
        _say(f"[seq_used] {name} dk_mode={dk_mode} {variant}")
        idx = x.idx.copy()
        if variant == "garbage_in_unused_rows":
            idx = cleaned.copy()
            unused = row_in >= used_q[row_b]
            idx[unused] = 1_000_000
        ti = torch.from_numpy(idx).cuda()
        md = slikl.slikl_grad_metadata(t["q"], t["k"], ti, dk_mode=dk_mode, **max_seqlens(x), **kw)
        kl = torch.full(t["p"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
        dq, dk, dw, y = slikl.slikl_grad(t["q"], t["k"], t["w"], ti, t["p"], metadata=md, dk_mode=dk_mode,
                                         kl_loss=kl, **max_seqlens(x), **kw)
        torch.cuda.synchronize()
        flagged = bool(int(md[8].item()) & 4)
        used_rows = row_in < used_q[row_b]
        past = bool(np.any((cleaned != x.idx)[used_rows]))     # a used row names a key past the used ones
        assert flagged == (variant == "past_used_keys" and past)
        got = dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(), dw=dw.cpu().numpy(),
                   softmax_out=y.cpu().numpy())
        check_close(got, ref, label=f"{name} {dk_mode} {variant}")
        kg = kl.cpu().numpy().reshape(kref.shape).astype(np.float64)
        assert np.max(np.abs(kg - kref) - 1e-4 * (1 + np.abs(kref))) <= 0


@pytest.mark.parametrize("dk_mode,det", [("dense", False), ("sorted", True), ("scatter", True)])
def test_graph_capture_replays_match_eager(dk_mode, det):
    """The metadata pre-pass and slikl_grad captured into one HIP graph: every replay
    (eager fills of the outputs and synchronisations in between) gives the eager call's
    results bit for bit (strategies with reproducible dk)."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    x = make_inputs(SMALL["hp64_d128_ragged"])
    t = to_device(x)
    kw = dict(dk_mode=dk_mode, deterministic=det)
    desc = slikl.make_desc(t["q"], t["k"], t["idx"], **kw)
    ws = torch.empty(slikl.slikl_grad_workspace_size(desc), dtype=torch.uint8, device="cuda")
    md = torch.empty(slikl.METADATA_INTS, dtype=torch.int32, device="cuda")
    out = (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["w"]),
           torch.empty_like(t["p"]))

    def call():
        slikl.slikl_grad_metadata(t["q"], t["k"], t["idx"], metadata=md, workspace=ws, **kw)
        slikl.slikl_grad(t["q"], t["k"], t["w"], t["idx"], t["p"], metadata=md, workspace=ws, out=out, **kw)

    _say(f"[graph] {dk_mode} det={det}")
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in out]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        for o in out:
            o.fill_(7)
        ws.fill_(3)                     # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dw", "softmax_out"), out, eager):
            assert torch.equal(a, b), (i, name)
    check_close(dict(dq=eager[0].float().cpu().numpy(), dk=eager[1].float().cpu().numpy(),
                     dw=eager[2].cpu().numpy(), softmax_out=eager[3].cpu().numpy()), oracle(x),
                label=f"graph {dk_mode}")
