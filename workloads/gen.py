"""Seeded input generators (no operator arithmetic lives here).

Every workload is described by a :class:`Workload` and expanded by
:func:`make_inputs` into host arrays:

* ``q``, ``k``: float32 values already rounded to the 16-bit storage type, and
  the raw 16-bit patterns (``q_bits``, ``k_bits``) that are uploaded to the GPU;
* ``w``: float32 head weights, ``p``: float32 target distribution
  (``attnSoftmaxL1Norm``), zero at padded slots;
* ``idx``: int32 top-k key indices, batch-relative, padded with -1;
* ``cu_q`` / ``cu_k``: int32 cumulative sequence lengths for TND sides.

Shapes follow the operator's BSND / TND layouts:
q [B,S1,N1,D] | [T1,N1,D], k [B,S2,N2,D] | [T2,N2,D], w [B,S1,N1] | [T1,N1],
idx / p [B,S1,N2,topk] | [T1,N2,topk].

Random streams: numpy ``Generator(PCG64)`` seeded from ``SeedSequence(seed)``
with one spawned child stream per tensor (q, k, w, idx, p, lengths), so that a
change in one recipe never shifts another tensor's draws.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BSND = "BSND"
TND = "TND"


# --------------------------------------------------------------------------
# 16-bit rounding of float32 draws (storage format only).
# --------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns ``(values_as_float32, bits_as_uint16)``.  Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    vals = (r.astype(np.uint32) << 16).view(np.float32)
    return vals.reshape(x.shape), r.reshape(x.shape)


def round_to_f16(x: np.ndarray):
    """Round float32 values to IEEE half (numpy's cast rounds to nearest even)."""
    h = np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    return h.astype(np.float32), h.view(np.uint16)


# --------------------------------------------------------------------------
# Workload description.
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layout: str = BSND                 # layout of both q and k
    batch: int = 1
    s1: int = 0                        # BSND query length per batch
    s2: int = 0                        # BSND key length per batch
    seqlens: Optional[tuple] = None    # TND: per-sequence lengths (q == k)
    seqlen_range: Optional[tuple] = None  # TND: draw `batch` lengths uniform in [lo, hi]
    n1: int = 8
    n2: int = 1
    d: int = 32
    topk: int = 16
    dtype: str = "bf16"                # "bf16" | "f16"
    q_var: float = 1.0
    k_var: float = 1.0
    w_var: float = 0.5
    index_mode: str = "causal"         # "causal" | "sink_zipf" | "random"
    q_offset: int = 0                  # query t sits at key position t + q_offset
    invalid_frac: float = 0.0          # fraction of -1 slots ("sink_zipf" / "random")
    sink_frac: float = 0.3             # "sink_zipf": share of valid slots from the sink
    sink_keys: int = 64
    zipf_s: float = 1.1
    duplicates: bool = False           # "random": draw with replacement
    p_mode: str = "softmax"            # "softmax" | "dirichlet"
    p_var: float = 1.0                 # softmax logits ~ N(0, p_var)
    p_alpha: float = 0.1               # dirichlet concentration
    deterministic: bool = False
    seed: int = 0
    k_outliers: int = 0                # key rows (of the flattened [T2, N2]) scaled up
    k_outlier_scale: float = 100.0     # their factor, applied before the 16-bit rounding

    @property
    def flops_per_token(self) -> int:
        """Nominal MFMA work per query token: three N1 x D x topk contractions."""
        return 6 * self.n1 * self.d * self.topk


@dataclasses.dataclass
class Inputs:
    wl: Workload
    layout_q: str
    layout_k: str
    batch: int
    q: np.ndarray
    k: np.ndarray
    q_bits: np.ndarray
    k_bits: np.ndarray
    w: np.ndarray
    idx: np.ndarray
    p: np.ndarray
    cu_q: Optional[np.ndarray]
    cu_k: Optional[np.ndarray]
    s1: int                      # BSND: S1; TND: T1
    s2: int                      # BSND: S2; TND: T2
    max_seqlen_q: int
    max_seqlen_k: int

    @property
    def t1(self) -> int:
        return int(self.q.shape[0] * (self.q.shape[1] if self.layout_q == BSND else 1))

    @property
    def t2(self) -> int:
        return int(self.k.shape[0] * (self.k.shape[1] if self.layout_k == BSND else 1))

    @property
    def valid_slots(self) -> int:
        return int((self.idx >= 0).sum())


# The five headline workloads (indexer backward shapes).
WORKLOADS = {
    "tiny_causal": Workload(
        name="tiny_causal", layout=BSND, batch=1, s1=128, s2=128, n1=8, n2=1, d=32,
        topk=16, dtype="bf16", w_var=0.5, index_mode="causal", p_var=1.0, seed=1000),
    "dsv32_indexer": Workload(
        name="dsv32_indexer", layout=BSND, batch=1, s1=4096, s2=4096, n1=64, n2=1,
        d=128, topk=2048, dtype="bf16", w_var=1.0 / 8, index_mode="causal",
        p_var=2.0, seed=1001),
    "varlen_tnd": Workload(
        name="varlen_tnd", layout=TND, batch=8, seqlen_range=(512, 8192), n1=64, n2=1,
        d=128, topk=2048, dtype="f16", w_var=1.0 / 8, index_mode="causal",
        p_mode="dirichlet", p_alpha=0.1, seed=1002),
    "long_context": Workload(
        name="long_context", layout=BSND, batch=1, s1=8192, s2=131072, n1=32, n2=1,
        d=128, topk=2048, dtype="bf16", w_var=1.0 / 8, index_mode="causal",
        q_offset=131072 - 8192, p_var=2.0, seed=1003),
    "contention_det": Workload(
        name="contention_det", layout=BSND, batch=4, s1=8192, s2=8192, n1=16, n2=1,
        d=128, topk=512, dtype="bf16", w_var=0.25, index_mode="sink_zipf",
        invalid_frac=0.1, sink_frac=0.3, sink_keys=64, zipf_s=1.1, p_var=1.0,
        deterministic=True, seed=1004),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


# --------------------------------------------------------------------------
# Index-list recipes.
# --------------------------------------------------------------------------
def _zipf_table(n: int, s: float) -> np.ndarray:
    wts = (np.arange(1, n + 1, dtype=np.float64)) ** (-s)
    return np.cumsum(wts)


def _rows_indices(wl: Workload, rng: np.random.Generator, positions: np.ndarray,
                  key_len: int, zipf_cdf: Optional[np.ndarray]) -> np.ndarray:
    """Index lists for rows whose query sits at the given key positions."""
    topk = wl.topk
    out = np.full((positions.shape[0], topk), -1, dtype=np.int32)
    for r, pos in enumerate(positions):
        hi = int(min(pos, key_len - 1))          # keys [0, hi] are visible
        if hi < 0:
            continue
        if wl.index_mode == "causal":
            n = min(topk, hi + 1)
            out[r, :n] = rng.choice(hi + 1, size=n, replace=False)
        elif wl.index_mode == "sink_zipf":
            n_inv = int(round(wl.invalid_frac * topk))
            n_val = topk - n_inv
            n_sink = int(round(wl.sink_frac * n_val))
            n_zipf = n_val - n_sink
            sink = rng.integers(0, min(wl.sink_keys - 1, hi) + 1, size=n_sink)
            u = rng.random(n_zipf) * zipf_cdf[hi]
            zipf = np.minimum(np.searchsorted(zipf_cdf[: hi + 1], u, side="right"), hi)
            vals = np.concatenate([sink, zipf]).astype(np.int32)
            rng.shuffle(vals)
            slots = np.sort(rng.choice(topk, size=n_val, replace=False))
            out[r, slots] = vals
        elif wl.index_mode == "random":
            n_inv = int(round(wl.invalid_frac * topk))
            n_val = topk - n_inv
            if not wl.duplicates:
                n_val = min(n_val, hi + 1)
                vals = rng.choice(hi + 1, size=n_val, replace=False).astype(np.int32)
            else:
                vals = rng.integers(0, hi + 1, size=n_val).astype(np.int32)
            slots = np.sort(rng.choice(topk, size=n_val, replace=False))
            out[r, slots] = vals
        else:
            raise ValueError(f"unknown index_mode {wl.index_mode!r}")
    return out


def _target_dist(wl: Workload, rng: np.random.Generator, idx: np.ndarray) -> np.ndarray:
    """Target distribution over the valid slots of each row (0 at -1 slots)."""
    valid = idx >= 0
    p = np.zeros(idx.shape, dtype=np.float64)
    flat_valid = valid.reshape(-1, idx.shape[-1])
    flat_p = p.reshape(-1, idx.shape[-1])
    if wl.p_mode == "softmax":
        logits = rng.normal(0.0, np.sqrt(wl.p_var), size=flat_p.shape)
        logits = np.where(flat_valid, logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        e = np.where(flat_valid, np.exp(logits - mx), 0.0)
        z = e.sum(axis=1, keepdims=True)
        flat_p[:] = np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)
    elif wl.p_mode == "dirichlet":
        for r in range(flat_p.shape[0]):
            n = int(flat_valid[r].sum())
            if n:
                flat_p[r, flat_valid[r]] = rng.dirichlet(np.full(n, wl.p_alpha))
    else:
        raise ValueError(f"unknown p_mode {wl.p_mode!r}")
    return p.astype(np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Expand a workload into seeded host arrays (see module docstring)."""
    ss = np.random.SeedSequence(wl.seed if seed is None else seed)
    # spawned children depend only on their index: adding the seventh (outlier rows)
    # leaves the draws of the first six unchanged
    rq, rk, rw, ri, rp, rl, ro = (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(7))
    rnd = round_to_bf16 if wl.dtype == "bf16" else round_to_f16

    if wl.layout == BSND:
        B = wl.batch
        q_shape = (B, wl.s1, wl.n1, wl.d)
        k_shape = (B, wl.s2, wl.n2, wl.d)
        qlens = [wl.s1] * B
        klens = [wl.s2] * B
        cu_q = cu_k = None
    else:
        if wl.seqlens is not None:
            lens = list(wl.seqlens)
        else:
            lo, hi = wl.seqlen_range
            lens = [int(x) for x in rl.integers(lo, hi + 1, size=wl.batch)]
        B = len(lens)
        qlens = klens = lens
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        cu_q = cu.copy()
        cu_k = cu.copy()
        q_shape = (int(cu[-1]), wl.n1, wl.d)
        k_shape = (int(cu[-1]), wl.n2, wl.d)

    q, q_bits = rnd(rq.normal(0.0, np.sqrt(wl.q_var), size=q_shape).astype(np.float32))
    kf = rk.normal(0.0, np.sqrt(wl.k_var), size=k_shape).astype(np.float32)
    if wl.k_outliers > 0:
        flat = kf.reshape(-1, wl.d)
        pick = ro.choice(flat.shape[0], size=min(wl.k_outliers, flat.shape[0]), replace=False)
        flat[pick] *= np.float32(wl.k_outlier_scale)
    k, k_bits = rnd(kf)
    w = rw.normal(0.0, np.sqrt(wl.w_var), size=q_shape[:-1]).astype(np.float32)

    zipf_cdf = _zipf_table(max(klens), wl.zipf_s) if wl.index_mode == "sink_zipf" else None
    rows = []
    for b in range(B):
        pos = np.arange(qlens[b], dtype=np.int64) + wl.q_offset
        per_group = [_rows_indices(wl, ri, pos, klens[b], zipf_cdf) for _ in range(wl.n2)]
        rows.append(np.stack(per_group, axis=1))          # [S1_b, N2, topk]
    if wl.layout == BSND:
        idx = np.stack(rows, axis=0)                       # [B, S1, N2, topk]
    else:
        idx = np.concatenate(rows, axis=0)                 # [T1, N2, topk]
    p = _target_dist(wl, rp, idx)

    return Inputs(
        wl=wl, layout_q=wl.layout, layout_k=wl.layout, batch=B, q=q, k=k,
        q_bits=q_bits, k_bits=k_bits, w=w, idx=np.ascontiguousarray(idx, dtype=np.int32),
        p=p, cu_q=cu_q, cu_k=cu_k,
        s1=wl.s1 if wl.layout == BSND else int(q_shape[0]),
        s2=wl.s2 if wl.layout == BSND else int(k_shape[0]),
        max_seqlen_q=max(qlens) if qlens else 0,
        max_seqlen_k=max(klens) if klens else 0,
    )


# --------------------------------------------------------------------------
# Main-attention inputs of the target distribution p (attnSoftmaxL1Norm).
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AttnPWorkload:
    """Main-attention queries / keys and the index lists p is taken at.  The
    index lists follow the recipe of ``index`` (an indexer Workload: layout,
    lengths, key heads, topk and index mode); nm / dm are the main attention's
    query heads and head dim."""
    name: str
    index: Workload
    nm: int = 128
    dm: int = 576
    scale: float = 1.0 / 192 ** 0.5
    q_var: float = 1.0
    k_var: float = 1.0
    seed: int = 0


@dataclasses.dataclass
class AttnPInputs:
    wl: AttnPWorkload
    layout_q: str
    layout_k: str
    batch: int
    qm: np.ndarray              # float32 values of the 16-bit qm
    km: np.ndarray
    qm_bits: np.ndarray
    km_bits: np.ndarray
    idx: np.ndarray
    cu_q: Optional[np.ndarray]
    cu_k: Optional[np.ndarray]

    @property
    def t1(self) -> int:
        return int(self.idx.reshape(-1, self.idx.shape[-2], self.idx.shape[-1]).shape[0])

    @property
    def valid_slots(self) -> int:
        return int((self.idx >= 0).sum())


def make_attn_p_inputs(wl: AttnPWorkload) -> AttnPInputs:
    """Index lists (and lengths) exactly as make_inputs(wl.index) draws them, plus
    main-attention queries [.., nm, dm] and keys [.., N2, dm] from their own streams."""
    base = make_inputs(wl.index)
    rq, rk = (np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(wl.seed).spawn(2))
    rnd = round_to_bf16 if wl.index.dtype == "bf16" else round_to_f16
    lead_q = base.q.shape[:-2]
    lead_k = base.k.shape[:-2]
    n2 = base.k.shape[-2]
    qm, qm_bits = rnd(rq.normal(0.0, np.sqrt(wl.q_var), size=lead_q + (wl.nm, wl.dm)).astype(np.float32))
    km, km_bits = rnd(rk.normal(0.0, np.sqrt(wl.k_var), size=lead_k + (n2, wl.dm)).astype(np.float32))
    return AttnPInputs(wl=wl, layout_q=base.layout_q, layout_k=base.layout_k, batch=base.batch, qm=qm, km=km,
                       qm_bits=qm_bits, km_bits=km_bits, idx=base.idx, cu_q=base.cu_q, cu_k=base.cu_k)


# The main-attention workload of p at the DeepSeek-V3.2 indexer's shape: 128 query heads
# sharing one key head, head dim 576 (a 512-wide latent plus 64 rotary dims), softmax
# scale 1/sqrt(192), over the DeepSeek-shaped indexer's causal top-2048 lists.
ATTN_P_WORKLOADS = {
    "attn_p_dsv32": AttnPWorkload(name="attn_p_dsv32", index=WORKLOADS["dsv32_indexer"], nm=128, dm=576,
                                  scale=1.0 / 192 ** 0.5, seed=2001),
}


# --------------------------------------------------------------------------
# Inputs of the dense sibling operator: no index lists; p is dense over the key
# positions and nonzero on the keys the mask shows.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DenseInputs:
    wl: Workload
    mask_mode: int
    layout_q: str
    layout_k: str
    batch: int
    q: np.ndarray
    k: np.ndarray
    q_bits: np.ndarray
    k_bits: np.ndarray
    w: np.ndarray
    p: np.ndarray                # [.., N2, L]
    cu_q: Optional[np.ndarray]
    cu_k: Optional[np.ndarray]
    max_seqlen_q: int
    max_seqlen_k: int

    @property
    def t1(self) -> int:
        return int(self.p.reshape(-1, self.p.shape[-2], self.p.shape[-1]).shape[0])

    @property
    def visible(self) -> int:
        return int((self.p > 0).sum())


def make_dense_inputs(wl: Workload, mask_mode: int) -> DenseInputs:
    """q, k, w (and TND lengths) as make_inputs draws them; p from the workload's
    p recipe over each row's visible keys (maskMode 0: all keys of the batch; 3: keys
    j <= t + S2_b - S1_b), 0 elsewhere.  The dense axis L is the longest key sequence."""
    base = make_inputs(dataclasses.replace(wl, topk=1, index_mode="causal"))
    rp = np.random.Generator(np.random.PCG64(np.random.SeedSequence(wl.seed + 7919)))
    n2 = base.k.shape[-2]
    if base.layout_q == BSND:
        qlens = [base.q.shape[1]] * base.batch
        klens = [base.k.shape[1]] * base.batch
    else:
        qlens = list(np.diff(base.cu_q))
        klens = list(np.diff(base.cu_k))
    L = max(klens) if klens else 0
    rows = []
    for b in range(base.batch):
        s1b, s2b = int(qlens[b]), int(klens[b])
        pb = np.zeros((s1b, n2, L))
        for t in range(s1b):
            n = s2b if mask_mode == 0 else max(0, min(s2b, t + s2b - s1b + 1))
            if n == 0:
                continue
            if wl.p_mode == "dirichlet":
                for g in range(n2):
                    pb[t, g, :n] = rp.dirichlet(np.full(n, wl.p_alpha))
            else:
                lg = rp.normal(0.0, np.sqrt(wl.p_var), size=(n2, n))
                e = np.exp(lg - lg.max(-1, keepdims=True))
                pb[t, :, :n] = e / e.sum(-1, keepdims=True)
        rows.append(pb)
    if base.layout_q == BSND:
        p = np.stack(rows, axis=0)
    else:
        p = np.concatenate(rows, axis=0) if rows else np.zeros((0, n2, L))
    return DenseInputs(wl=wl, mask_mode=mask_mode, layout_q=base.layout_q, layout_k=base.layout_k,
                       batch=base.batch, q=base.q, k=base.k, q_bits=base.q_bits, k_bits=base.k_bits, w=base.w,
                       p=p.astype(np.float32), cu_q=base.cu_q, cu_k=base.cu_k,
                       max_seqlen_q=max(qlens) if qlens else 0, max_seqlen_k=L)


# The dense operator at the DeepSeek-shaped indexer's width over 2048-key rows (the
# longest row the fused kernel holds): two sequences of 2048, rightDownCausal mask.
DENSE_WORKLOADS = {
    "dense_dsv32_2k": (Workload(name="dense_dsv32_2k", layout=BSND, batch=2, s1=2048, s2=2048, n1=64, n2=1, d=128,
                                topk=1, dtype="bf16", w_var=1.0 / 8, p_var=2.0, seed=3001), 3),
}
