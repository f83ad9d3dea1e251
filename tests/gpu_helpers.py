"""Shared helpers of the GPU parity tests: upload seeded inputs, call the HIP
path through the C ABI binding, compare with the fp64 oracle.

Tolerances (from the operator's accuracy targets):
  softmax_out  max |gpu - ref| <= 1e-5
  dw           max |gpu - ref| / max |ref| <= 1e-3
  dq, dk       |gpu - ref| <= 1e-3 + 2e-2 |ref| elementwise (16-bit outputs)
"""
from __future__ import annotations

import numpy as np

Y_ATOL = 1e-5
DW_REL = 1e-3
G_ATOL = 1e-3
G_RTOL = 2e-2


def to_device(x, device="cuda"):
    import torch
    tdt = torch.bfloat16 if x.wl.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(device)

    t = dict(
        q=b16(x.q_bits), k=b16(x.k_bits),
        w=torch.from_numpy(np.ascontiguousarray(x.w, dtype=np.float32)).to(device),
        idx=torch.from_numpy(np.ascontiguousarray(x.idx, dtype=np.int32)).to(device),
        p=torch.from_numpy(np.ascontiguousarray(x.p, dtype=np.float32)).to(device),
        cu_q=None if x.cu_q is None else torch.from_numpy(x.cu_q.astype(np.int32)).to(device),
        cu_k=None if x.cu_k is None else torch.from_numpy(x.cu_k.astype(np.int32)).to(device),
    )
    return t


def max_seqlens(x):
    """Longest sequence of each TND side (host-known from the generator), 0 for BSND."""
    def mx(cu):
        return int(np.diff(np.asarray(cu)).max()) if cu is not None and len(cu) > 1 else 0
    return dict(max_seqlen_q=mx(x.cu_q) if x.layout_q == "TND" else 0,
                max_seqlen_k=mx(x.cu_k) if x.layout_k == "TND" else 0)


def run_gpu(x, t=None, kl=False, **kw):
    """Call slikl_grad; returns numpy fp32/fp64 arrays (dq, dk, dw, y, and with
    kl=True the per-unit KL output).  TND sides pass their longest sequence unless
    the caller gives max_seqlen_q / _k."""
    import torch
    import sparse_attention_indexer_token_amd as slikl
    if t is None:
        t = to_device(x)
    for key, val in max_seqlens(x).items():
        kw.setdefault(key, val)
    if kl:
        # filled with NaN first: every unit must be written
        kw["kl_loss"] = torch.full(t["p"].shape[:-1], float("nan"), dtype=torch.float32, device=t["p"].device)
    dq, dk, dw, y = slikl.slikl_grad(
        t["q"], t["k"], t["w"], t["idx"], t["p"], layout_q=x.layout_q, layout_k=x.layout_k,
        cu_seqlens_q=t["cu_q"], cu_seqlens_k=t["cu_k"],
        deterministic=kw.pop("deterministic", x.wl.deterministic), **kw)
    torch.cuda.synchronize()
    out = dict(dq=dq.float().cpu().numpy(), dk=dk.float().cpu().numpy(),
               dw=dw.cpu().numpy(), softmax_out=y.cpu().numpy())
    if kl:
        out["kl_loss"] = kw["kl_loss"].cpu().numpy()
    return out


def oracle(x, rows=None):
    from oracle import slikl_grad_ref
    return slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                          cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows)


def check_close(got, ref, *, rows=None, what=("dq", "dk", "dw", "softmax_out"), label=""):
    """Assert the tolerances; `rows` restricts dq / dw / softmax_out to those flat rows."""
    msgs = []
    for name in what:
        g = np.asarray(got[name], dtype=np.float64)
        r = np.asarray(ref[name], dtype=np.float64)
        if rows is not None and name != "dk":
            lead = g.shape[:-2] if name != "dw" else g.shape[:-1]
            n_lead = int(np.prod(lead[:2])) if len(lead) >= 2 else int(lead[0])
            g = g.reshape((n_lead,) + g.shape[len(lead):])[rows]
            r = r.reshape((n_lead,) + r.shape[len(lead):])[rows]
        if g.size == 0:
            continue
        err = np.abs(g - r)
        if name == "softmax_out":
            ok = err.max() <= Y_ATOL
            msgs.append(f"{name}: max abs {err.max():.3e}")
        elif name == "dw":
            scale = max(np.abs(r).max(), 1e-30)
            ok = err.max() / scale <= DW_REL
            msgs.append(f"{name}: max rel {err.max() / scale:.3e}")
        else:
            bound = G_ATOL + G_RTOL * np.abs(r)
            ok = bool(np.all(err <= bound))
            worst = np.unravel_index(np.argmax(err - bound), err.shape)
            msgs.append(f"{name}: worst excess {float((err - bound)[worst]):.3e} at {worst} "
                        f"(got {g[worst]:.5g} ref {r[worst]:.5g})")
        assert ok, f"{label} {' | '.join(msgs)}"
    return msgs


def keys_with_few_refs(x, max_rows=8, want=16, rng=None):
    """Flat key rows whose referencing query rows are few; returns {key: rows}."""
    n2 = x.idx.shape[-2]
    topk = x.idx.shape[-1]
    idx = x.idx.reshape(-1, n2, topk)
    T1 = idx.shape[0]
    if x.layout_q == "BSND":
        S1 = x.q.shape[1]
        qbatch = np.arange(T1) // S1
    else:
        qbatch = np.searchsorted(x.cu_q, np.arange(T1), side="right") - 1
    if x.layout_k == "BSND":
        kbase = qbatch * x.k.shape[1]
    else:
        kbase = x.cu_k[qbatch]
    flat = np.where(idx >= 0, idx + kbase[:, None, None], -1).reshape(T1, -1)
    rows = np.broadcast_to(np.arange(T1)[:, None], flat.shape)
    v = flat >= 0
    pair = np.unique(flat[v].astype(np.int64) * T1 + rows[v])      # unique (key, row)
    keys, rws = pair // T1, pair % T1
    uk, start, cnt = np.unique(keys, return_index=True, return_counts=True)
    ok = np.flatnonzero(cnt <= max_rows)
    rng = rng or np.random.default_rng(0)
    pick = rng.permutation(ok)[:want]
    return {int(uk[i]): rws[start[i]:start[i] + cnt[i]] for i in pick}
