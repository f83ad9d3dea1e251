"""The seeded generators: determinism, shapes and the structure each recipe promises."""
import numpy as np

from workloads import WORKLOADS, Workload, make_inputs, round_to_bf16


def test_same_seed_same_bytes():
    a = make_inputs(WORKLOADS["tiny_causal"])
    b = make_inputs(WORKLOADS["tiny_causal"])
    for name in ("q_bits", "k_bits", "w", "idx", "p"):
        assert np.array_equal(getattr(a, name), getattr(b, name))


def test_tiny_causal_structure():
    x = make_inputs(WORKLOADS["tiny_causal"])
    assert x.q.shape == (1, 128, 8, 32) and x.k.shape == (1, 128, 1, 32)
    assert x.idx.shape == (1, 128, 1, 16)
    assert x.valid_slots == 1928
    for t in range(128):
        row = x.idx[0, t, 0]
        n = min(16, t + 1)
        assert np.all(row[n:] == -1)
        v = row[:n]
        assert len(set(v.tolist())) == n and v.min() >= 0 and v.max() <= t
        assert abs(x.p[0, t, 0, :n].sum() - 1) < 1e-5 and np.all(x.p[0, t, 0, n:] == 0)


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5], dtype=np.float32)
    r, bits = round_to_bf16(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa is 1.0
    assert r.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5]
    assert bits[0] == 0x3F80


def test_varlen_tnd_small():
    wl = Workload(name="v", layout="TND", batch=3, seqlen_range=(4, 9), n1=4, n2=1, d=8,
                  topk=5, dtype="f16", p_mode="dirichlet", seed=3)
    x = make_inputs(wl)
    assert x.cu_q[0] == 0 and np.all(np.diff(x.cu_q) >= 4)
    for b in range(3):
        for t in range(x.cu_q[b + 1] - x.cu_q[b]):
            row = x.idx[x.cu_q[b] + t, 0]
            v = row[row >= 0]
            assert v.size == min(5, t + 1) and v.max() <= t
            s = x.p[x.cu_q[b] + t, 0].sum()
            assert abs(s - 1) < 1e-5


def test_sink_zipf_small():
    wl = Workload(name="c", batch=2, s1=100, s2=100, n1=4, n2=1, d=8, topk=50,
                  index_mode="sink_zipf", invalid_frac=0.1, sink_frac=0.3, sink_keys=8, seed=4)
    x = make_inputs(wl)
    inv = (x.idx == -1).sum(-1)
    assert np.all(inv == 5)
    for t in range(100):
        row = x.idx[0, t, 0]
        assert row[row >= 0].max() <= t
    # the first keys are hot
    counts = np.bincount(x.idx[x.idx >= 0].ravel(), minlength=100)
    assert counts[:8].sum() > 0.3 * counts.sum()
