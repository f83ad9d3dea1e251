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
                          cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows, kink=True)


def check_close(got, ref, *, rows=None, what=("dq", "dk", "dw", "softmax_out"), label="",
                y_logit_scaled=False):
    """Assert the tolerances; `rows` restricts dq / dw / softmax_out to those flat rows.

    dq and dk elements also allow the oracle's kink allowance (``dq_kink`` /
    ``dk_kink`` when present): the change that deciding 1[S > 0] the other way at
    scores within fp32 rounding of 0 makes.  With y_logit_scaled, softmax_out
    allows 1e-5 + 2 u M y elementwise, u = 2^-24 and M the unit's logit scale
    (max_s sum_h |w_h S_hs|): the first-order change of a softmax whose logits
    carry errors up to u M, for inputs whose logits are far larger than the
    pages' workloads have."""
    msgs = []

    def pick(a, name, trail):
        # flat query rows of an output whose last `trail` axes are per row
        a = np.asarray(a, dtype=np.float64)
        if rows is None or name == "dk":
            return a
        return a.reshape((-1,) + a.shape[a.ndim - trail:])[rows]

    for name in what:
        trail = 1 if name == "dw" else 2
        g = pick(got[name], name, trail)
        r = pick(ref[name], name, trail).reshape(g.shape)
        if g.size == 0:
            continue
        err = np.abs(g - r)
        if name == "softmax_out":
            if y_logit_scaled:
                m = pick(ref["logit_scale"], name, 1).reshape(g.shape[:-1])[..., None]
                bound = Y_ATOL + 2.0 * 2.0 ** -24 * m * np.abs(r)
                ok = bool(np.all(err <= bound))
                msgs.append(f"{name}: max abs {err.max():.3e}, worst err/bound {float((err / bound).max()):.3f}")
            else:
                ok = err.max() <= Y_ATOL
                msgs.append(f"{name}: max abs {err.max():.3e}")
        elif name == "dw":
            # the bound reads max |err| / max |ref| over the tensor; a per-row reading
            # (|err_row| / |ref_row| in the 2-norm, over rows whose norm exceeds 1e-3 of
            # the largest) is checked beside it
            scale = max(np.abs(r).max(), 1e-30)
            ok = err.max() / scale <= DW_REL
            en = np.sqrt((err.reshape(-1, err.shape[-1]) ** 2).sum(-1))
            rn = np.sqrt((r.reshape(-1, r.shape[-1]) ** 2).sum(-1))
            big = rn > 1e-3 * max(rn.max(), 1e-30)
            row_rel = float((en[big] / rn[big]).max()) if big.any() else 0.0
            ok = ok and row_rel <= DW_REL
            msgs.append(f"{name}: max rel {err.max() / scale:.3e}, worst row rel {row_rel:.3e}")
        else:
            bound = G_ATOL + G_RTOL * np.abs(r)
            if f"{name}_kink" in ref:
                bound = bound + pick(ref[f"{name}_kink"], name, trail).reshape(g.shape)
            ok = bool(np.all(err <= bound))
            worst = np.unravel_index(np.argmax(err - bound), err.shape)
            msgs.append(f"{name}: worst excess {float((err - bound)[worst]):.3e} at {worst} "
                        f"(got {g[worst]:.5g} ref {r[worst]:.5g})")
        assert ok, f"{label} {' | '.join(msgs)}"
    return msgs
