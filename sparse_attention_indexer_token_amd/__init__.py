"""Sparse lightning-indexer KL-loss backward on AMD MI355X (gfx950).

Thin PyTorch binding over the C ABI of ``libslikl.so`` (include/slikl.h).
The functions below carry the C names and only marshal arguments: they read
shapes from the tensors, allocate outputs / workspace with torch on the
tensors' device and pass raw device pointers and the current HIP stream.

    dq, dk, dw, softmax_out = slikl_grad(q, k, w, sparse_indices, p)

Shapes (BSND | TND):
    q [B,S1,N1,D] | [T1,N1,D] (bf16 or fp16), k [B,S2,N2,D] | [T2,N2,D] (same dtype),
    w [B,S1,N1] | [T1,N1] fp32, sparse_indices / p [B,S1,N2,topk] | [T1,N2,topk]
    (int32 / fp32).  TND sides need int32 cumulative lengths (B+1 entries).
"""
from __future__ import annotations

from typing import Optional

from . import _native
from ._native import (  # noqa: F401
    EXPORTS, LAYOUT, METADATA_HEADER, METADATA_INTS, MAX_PARTS, STATIC_SCRATCH_BYTES, SliklDesc,
    SliklError, UNIT_OVERHEAD, UNIT_OVERHEAD_DENSE, load,
)

__all__ = ["slikl_grad", "slikl_grad_profiled", "slikl_grad_metadata", "slikl_grad_workspace_size",
           "slikl_grad_parts", "slikl_grad_unit_overhead", "slikl_grad_dk_strategy", "slikl_status_string",
           "slikl_grad_noalloc", "slikl_grad_noalloc_strategy", "slikl_attn_softmax_l1norm",
           "slikl_dense_grad", "slikl_dense_grad_profiled", "slikl_dense_grad_metadata",
           "slikl_dense_grad_workspace_size", "make_dense_desc", "make_desc", "SliklDesc", "SliklError"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _native.DTYPE["bf16"]
    if t.dtype == torch.float16:
        return _native.DTYPE["f16"]
    raise TypeError(f"q/k must be bfloat16 or float16, got {t.dtype}")


def make_desc(q, k, sparse_indices, *, layout_q: str = "BSND", layout_k: str = "BSND",
              cu_seqlens_q=None, cu_seqlens_k=None, deterministic: bool = False,
              num_parts: int = 0, split_mode: str = "weighted",
              dk_mode: str = "auto", max_seqlen_q: int = 0, max_seqlen_k: int = 0,
              seq_used_q=None, seq_used_k=None) -> SliklDesc:
    """Build the C descriptor from tensor shapes (no device access).

    For a TND side, ``max_seqlen_q`` / ``max_seqlen_k`` may give its longest sequence
    (0 = not given); the dense dK strategy needs them for TND inputs.
    ``seq_used_q`` / ``seq_used_k`` (TND sides, optional int32 [B] device tensors):
    each batch's used length; rows past it take no part, keys past it are out of
    range."""
    if layout_q not in LAYOUT or layout_k not in LAYOUT:
        raise ValueError("layouts must be 'BSND' or 'TND'")
    if layout_q == "BSND":
        if q.dim() != 4:
            raise ValueError("BSND q must be [B,S1,N1,D]")
        batch, s1, n1, d = q.shape
    else:
        if q.dim() != 3 or cu_seqlens_q is None:
            raise ValueError("TND q must be [T1,N1,D] with cu_seqlens_q")
        s1, n1, d = q.shape
        batch = cu_seqlens_q.numel() - 1
    if layout_k == "BSND":
        if k.dim() != 4:
            raise ValueError("BSND k must be [B,S2,N2,D]")
        kb, s2, n2, dk_ = k.shape
        if layout_q == "TND" and kb != batch:
            raise ValueError("batch of k does not match cu_seqlens_q")
        batch = kb if layout_q == "BSND" else batch
        if layout_q == "BSND" and kb != q.shape[0]:
            raise ValueError("q and k disagree on B")
    else:
        if k.dim() != 3 or cu_seqlens_k is None:
            raise ValueError("TND k must be [T2,N2,D] with cu_seqlens_k")
        s2, n2, dk_ = k.shape
        if cu_seqlens_k.numel() - 1 != batch:
            raise ValueError("cu_seqlens_k does not match the batch")
    if dk_ != d:
        raise ValueError("q and k disagree on D")
    desc = SliklDesc()
    desc.layout_q = LAYOUT[layout_q]
    desc.layout_k = LAYOUT[layout_k]
    desc.dtype = _dtype_code(q)
    desc.deterministic = 1 if deterministic else 0
    desc.batch, desc.s1, desc.s2 = int(batch), int(s1), int(s2)
    desc.n1, desc.n2, desc.d = int(n1), int(n2), int(d)
    desc.topk = int(sparse_indices.shape[-1])
    desc.cu_seqlens_q = cu_seqlens_q.data_ptr() if layout_q == "TND" else None
    desc.cu_seqlens_k = cu_seqlens_k.data_ptr() if layout_k == "TND" else None
    desc.num_parts = int(num_parts)
    desc.split_mode = _native.SPLIT[split_mode]
    desc.dk_mode = _native.DK_MODE[dk_mode]
    desc.max_seqlen_q = int(max_seqlen_q) if layout_q == "TND" else 0
    desc.max_seqlen_k = int(max_seqlen_k) if layout_k == "TND" else 0
    for name, t, lay in (("seq_used_q", seq_used_q, layout_q), ("seq_used_k", seq_used_k, layout_k)):
        if t is None:
            setattr(desc, name, None)
            continue
        if lay != "TND":
            raise ValueError(f"{name} applies to a TND side only")
        _check_tensor(name, t, _torch().int32, q.device, (desc.batch,))
        setattr(desc, name, t.data_ptr())
    return desc


def _check_tensor(name, t, dtype, device, shape=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def slikl_status_string(status: int) -> str:
    return _native.status_string(status)


def slikl_grad_workspace_size(desc: SliklDesc) -> int:
    return _native.workspace_size(desc)


def slikl_grad_parts(desc: SliklDesc) -> int:
    return _native.grad_parts(desc)


def slikl_grad_unit_overhead(desc: SliklDesc) -> int:
    """Per-unit overhead (valid-slot equivalents) of the weighted split for `desc`."""
    return _native.unit_overhead(desc)


def slikl_grad_dk_strategy(desc: SliklDesc) -> str:
    """The dK strategy ("scatter", "dense" or "sorted") a call with `desc` runs."""
    return _native.dk_strategy(desc)


def slikl_grad_metadata(q, k, sparse_indices, *, layout_q="BSND", layout_k="BSND",
                        cu_seqlens_q=None, cu_seqlens_k=None, deterministic=False,
                        num_parts: int = 0, split_mode: str = "weighted", dk_mode: str = "auto",
                        max_seqlen_q: int = 0, max_seqlen_k: int = 0, metadata=None, workspace=None,
                        seq_used_q=None, seq_used_k=None):
    """Run the load-balancing metadata pre-pass; returns the int32 metadata tensor."""
    torch = _torch()
    desc = make_desc(q, k, sparse_indices, layout_q=layout_q, layout_k=layout_k,
                     cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                     deterministic=deterministic, num_parts=num_parts, split_mode=split_mode,
                     dk_mode=dk_mode, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                     seq_used_q=seq_used_q, seq_used_k=seq_used_k)
    dev = q.device
    _check_tensor("sparse_indices", sparse_indices, torch.int32, dev)
    nbytes = _native.workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if metadata is None:
        metadata = torch.empty(METADATA_INTS, dtype=torch.int32, device=dev)
    _check_tensor("metadata", metadata, torch.int32, dev, (METADATA_INTS,))
    _native.grad_metadata_raw(desc, sparse_indices.data_ptr(), metadata.data_ptr(),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream_handle(dev))
    return metadata


def slikl_grad(q, k, w, sparse_indices, attn_softmax_l1norm, *, layout_q="BSND", layout_k="BSND",
               cu_seqlens_q=None, cu_seqlens_k=None, deterministic: bool = False,
               metadata=None, num_parts: int = 0, split_mode: str = "weighted",
               dk_mode: str = "auto", max_seqlen_q: int = 0, max_seqlen_k: int = 0,
               workspace=None, out: Optional[tuple] = None, kl_loss=None,
               seq_used_q=None, seq_used_k=None):
    """Backward pass; returns (dq, dk, dw, softmax_out).

    ``out`` may hold preallocated (dq, dk, dw, softmax_out); ``workspace`` a
    uint8 device tensor of at least ``slikl_grad_workspace_size`` bytes.
    ``kl_loss`` (optional fp32 tensor shaped like softmax_out without its last
    axis) receives each (query row, key head) unit's KL(p || softmax_out); its sum
    is the loss.
    """
    return _grad(q, k, w, sparse_indices, attn_softmax_l1norm, layout_q=layout_q, layout_k=layout_k,
                 cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, deterministic=deterministic,
                 metadata=metadata, num_parts=num_parts, split_mode=split_mode, dk_mode=dk_mode,
                 max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                 workspace=workspace, out=out, kl_loss=kl_loss, seq_used_q=seq_used_q,
                 seq_used_k=seq_used_k, profiled=False)[0]


def slikl_grad_noalloc_strategy(desc: SliklDesc) -> str:
    """The dK strategy slikl_grad_noalloc runs for `desc`."""
    return _native.noalloc_strategy(desc)


def slikl_grad_noalloc(q, k, w, sparse_indices, attn_softmax_l1norm, *, out, layout_q="BSND",
                       layout_k="BSND", cu_seqlens_q=None, cu_seqlens_k=None,
                       deterministic: bool = False, metadata=None, num_parts: int = 0,
                       split_mode: str = "weighted", dk_mode: str = "auto", max_seqlen_q: int = 0,
                       max_seqlen_k: int = 0, kl_loss=None, seq_used_q=None, seq_used_k=None):
    """slikl_grad into the caller's preallocated ``out`` = (dq, dk, dw, softmax_out),
    with the library's fixed per-GPU workspace: neither this call nor the library
    allocates device memory.  Calls that overlap on one GPU race (one shared array)."""
    torch = _torch()
    desc = make_desc(q, k, sparse_indices, layout_q=layout_q, layout_k=layout_k,
                     cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                     deterministic=deterministic, num_parts=num_parts, split_mode=split_mode,
                     dk_mode=dk_mode, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                     seq_used_q=seq_used_q, seq_used_k=seq_used_k)
    dev = q.device
    rows = tuple(q.shape)[:-2]
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k", k, q.dtype, dev)
    _check_tensor("w", w, torch.float32, dev, rows + (desc.n1,))
    _check_tensor("sparse_indices", sparse_indices, torch.int32, dev, rows + (desc.n2, desc.topk))
    _check_tensor("attn_softmax_l1norm", attn_softmax_l1norm, torch.float32, dev,
                  rows + (desc.n2, desc.topk))
    if metadata is not None:
        _check_tensor("metadata", metadata, torch.int32, dev, (METADATA_INTS,))
    if kl_loss is not None:
        _check_tensor("kl_loss", kl_loss, torch.float32, dev, rows + (desc.n2,))
        desc.kl_loss = kl_loss.data_ptr()
    dq, dk, dw, y = out
    _check_tensor("dq", dq, q.dtype, dev, q.shape)
    _check_tensor("dk", dk, q.dtype, dev, k.shape)
    _check_tensor("dw", dw, torch.float32, dev, w.shape)
    _check_tensor("softmax_out", y, torch.float32, dev, attn_softmax_l1norm.shape)
    _native.grad_noalloc_raw(desc, q.data_ptr(), k.data_ptr(), w.data_ptr(), sparse_indices.data_ptr(),
                             attn_softmax_l1norm.data_ptr(), metadata.data_ptr() if metadata is not None else 0,
                             dq.data_ptr(), dk.data_ptr(), dw.data_ptr(), y.data_ptr(), _stream_handle(dev))
    return out


def slikl_grad_profiled(q, k, w, sparse_indices, attn_softmax_l1norm, **kw):
    """slikl_grad plus the per-phase milliseconds (HIP events on the current
    stream; blocks until the call has run).  Returns ((dq, dk, dw, softmax_out), {phase: ms})."""
    return _grad(q, k, w, sparse_indices, attn_softmax_l1norm, profiled=True, **kw)


def _grad(q, k, w, sparse_indices, attn_softmax_l1norm, *, layout_q="BSND", layout_k="BSND",
          cu_seqlens_q=None, cu_seqlens_k=None, deterministic: bool = False,
          metadata=None, num_parts: int = 0, split_mode: str = "weighted",
          dk_mode: str = "auto", max_seqlen_q: int = 0, max_seqlen_k: int = 0,
          workspace=None, out: Optional[tuple] = None, kl_loss=None, seq_used_q=None,
          seq_used_k=None, profiled: bool = False):
    torch = _torch()
    desc = make_desc(q, k, sparse_indices, layout_q=layout_q, layout_k=layout_k,
                     cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                     deterministic=deterministic, num_parts=num_parts, split_mode=split_mode,
                     dk_mode=dk_mode, max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k,
                     seq_used_q=seq_used_q, seq_used_k=seq_used_k)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    qs = tuple(q.shape)
    rows = qs[:-2]
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k", k, q.dtype, dev)
    _check_tensor("w", w, torch.float32, dev, rows + (desc.n1,))
    _check_tensor("sparse_indices", sparse_indices, torch.int32, dev, rows + (desc.n2, desc.topk))
    _check_tensor("attn_softmax_l1norm", attn_softmax_l1norm, torch.float32, dev,
                  rows + (desc.n2, desc.topk))
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu is not None:
            _check_tensor(name, cu, torch.int32, dev, (desc.batch + 1,))
    if metadata is not None:
        _check_tensor("metadata", metadata, torch.int32, dev, (METADATA_INTS,))
    if kl_loss is not None:
        _check_tensor("kl_loss", kl_loss, torch.float32, dev, rows + (desc.n2,))
        desc.kl_loss = kl_loss.data_ptr()
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dw = torch.empty_like(w)
        y = torch.empty_like(attn_softmax_l1norm)
    else:
        dq, dk, dw, y = out
        _check_tensor("dq", dq, q.dtype, dev, q.shape)
        _check_tensor("dk", dk, q.dtype, dev, k.shape)
        _check_tensor("dw", dw, torch.float32, dev, w.shape)
        _check_tensor("softmax_out", y, torch.float32, dev, attn_softmax_l1norm.shape)
    nbytes = _native.workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = (desc, q.data_ptr(), k.data_ptr(), w.data_ptr(), sparse_indices.data_ptr(),
            attn_softmax_l1norm.data_ptr(), metadata.data_ptr() if metadata is not None else 0,
            dq.data_ptr(), dk.data_ptr(), dw.data_ptr(), y.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(dev))
    if profiled:
        return (dq, dk, dw, y), _native.grad_profiled_raw(*args)
    _native.grad_raw(*args)
    return (dq, dk, dw, y), None


def slikl_attn_softmax_l1norm(q_main, k_main, sparse_indices, scale: float, *, lse=None, out=None,
                              layout_q: str = "BSND", layout_k: str = "BSND", cu_seqlens_q=None,
                              cu_seqlens_k=None):
    """The target distribution p (attnSoftmaxL1Norm) from the main attention: per
    (query row, key head) unit, the main-attention softmax probabilities of the
    unit's heads at its top-k slots, summed over the heads and L1-normalised.

    q_main [B,S1,Nm,Dm] | [T1,Nm,Dm], k_main [B,S2,N2,Dm] | [T2,N2,Dm] (bf16 / fp16),
    sparse_indices [.., N2, topk] int32; ``lse`` (optional fp32 [.., Nm]): each head's
    natural log-sum-exp over the keys the main attention normalised over (default:
    over the unit's valid slots).  Returns p [.., N2, topk] fp32 (or fills ``out``)."""
    torch = _torch()
    if layout_q not in LAYOUT or layout_k not in LAYOUT:
        raise ValueError("layouts must be 'BSND' or 'TND'")
    dev = q_main.device
    if layout_q == "BSND":
        if q_main.dim() != 4:
            raise ValueError("BSND q_main must be [B,S1,Nm,Dm]")
        batch, s1, nm, d = q_main.shape
    else:
        if q_main.dim() != 3 or cu_seqlens_q is None:
            raise ValueError("TND q_main must be [T1,Nm,Dm] with cu_seqlens_q")
        s1, nm, d = q_main.shape
        batch = cu_seqlens_q.numel() - 1
    if layout_k == "BSND":
        if k_main.dim() != 4 or (layout_q == "BSND" and k_main.shape[0] != batch):
            raise ValueError("BSND k_main must be [B,S2,N2,Dm] with the batch of q_main")
        kb, s2, n2, dk_ = k_main.shape
        batch = kb if layout_q == "BSND" else batch
    else:
        if k_main.dim() != 3 or cu_seqlens_k is None or cu_seqlens_k.numel() - 1 != batch:
            raise ValueError("TND k_main must be [T2,N2,Dm] with cu_seqlens_k of the batch")
        s2, n2, dk_ = k_main.shape
    if dk_ != d:
        raise ValueError("q_main and k_main disagree on Dm")
    rows = tuple(q_main.shape)[:-2]
    _check_tensor("q_main", q_main, q_main.dtype, dev)
    _check_tensor("k_main", k_main, q_main.dtype, dev)
    _check_tensor("sparse_indices", sparse_indices, torch.int32, dev, rows + (n2, sparse_indices.shape[-1]))
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, dev, rows + (nm,))
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu is not None:
            _check_tensor(name, cu, torch.int32, dev, (batch + 1,))
    desc = _native.SliklAttnPDesc()
    desc.layout_q, desc.layout_k = LAYOUT[layout_q], LAYOUT[layout_k]
    desc.dtype = _dtype_code(q_main)
    desc.reserved = 0
    desc.batch, desc.s1, desc.s2 = int(batch), int(s1), int(s2)
    desc.heads, desc.n2, desc.d = int(nm), int(n2), int(d)
    desc.topk = int(sparse_indices.shape[-1])
    desc.scale = float(scale)
    desc.cu_seqlens_q = cu_seqlens_q.data_ptr() if layout_q == "TND" else None
    desc.cu_seqlens_k = cu_seqlens_k.data_ptr() if layout_k == "TND" else None
    if out is None:
        out = torch.empty(sparse_indices.shape, dtype=torch.float32, device=dev)
    _check_tensor("p", out, torch.float32, dev, tuple(sparse_indices.shape))
    _native.attn_p_raw(desc, q_main.data_ptr(), k_main.data_ptr(), sparse_indices.data_ptr(),
                       lse.data_ptr() if lse is not None else 0, out.data_ptr(), _stream_handle(dev))
    return out


def make_dense_desc(q, k, attn_softmax_l1norm, *, mask_mode: int = 3, cmp_ratio: int = 1,
                    **kw) -> "_native.SliklDenseDesc":
    """Descriptor of the dense operator; ``kw`` as for make_desc (layouts, cuSeqLens,
    determinism, split, dK strategy, maxima).  The dense axis of p / softmax_out is
    the key length (S2, or max_seqlen_k for a TND k)."""
    desc = _native.SliklDenseDesc()
    desc.base = make_desc(q, k, attn_softmax_l1norm, **kw)   # (only the shape of p is read)
    desc.mask_mode = int(mask_mode)
    desc.cmp_ratio = int(cmp_ratio)
    return desc


def slikl_dense_grad_workspace_size(desc) -> int:
    return _native.dense_workspace_size(desc)


def slikl_dense_grad_metadata(q, k, attn_softmax_l1norm, *, mask_mode: int = 3, cmp_ratio: int = 1,
                              metadata=None, workspace=None, **kw):
    """The dense operator's load-balancing pre-pass; returns the int32 metadata."""
    torch = _torch()
    desc = make_dense_desc(q, k, attn_softmax_l1norm, mask_mode=mask_mode, cmp_ratio=cmp_ratio, **kw)
    dev = q.device
    nbytes = _native.dense_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if metadata is None:
        metadata = torch.empty(METADATA_INTS, dtype=torch.int32, device=dev)
    _check_tensor("metadata", metadata, torch.int32, dev, (METADATA_INTS,))
    _native.dense_metadata_raw(desc, metadata.data_ptr(), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream_handle(dev))
    return metadata


def slikl_dense_grad(q, k, w, attn_softmax_l1norm, *, mask_mode: int = 3, cmp_ratio: int = 1, metadata=None,
                     workspace=None, out=None, kl_loss=None, **kw):
    """Dense operator backward; returns (dq, dk, dw, softmax_out).  attn_softmax_l1norm
    and softmax_out are dense over the key positions: [.., N2, L]."""
    return _dense(q, k, w, attn_softmax_l1norm, mask_mode, cmp_ratio, metadata, workspace, out, kl_loss, kw,
                  profiled=False)[0]


def slikl_dense_grad_profiled(q, k, w, attn_softmax_l1norm, *, mask_mode: int = 3, cmp_ratio: int = 1,
                              metadata=None, workspace=None, out=None, kl_loss=None, **kw):
    return _dense(q, k, w, attn_softmax_l1norm, mask_mode, cmp_ratio, metadata, workspace, out, kl_loss, kw,
                  profiled=True)


def _dense(q, k, w, p, mask_mode, cmp_ratio, metadata, workspace, out, kl_loss, kw, profiled):
    torch = _torch()
    desc = make_dense_desc(q, k, p, mask_mode=mask_mode, cmp_ratio=cmp_ratio, **kw)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    rows = tuple(q.shape)[:-2]
    n2 = k.shape[-2]
    L = desc.base.s2 if kw.get("layout_k", "BSND") == "BSND" else desc.base.max_seqlen_k
    _check_tensor("q", q, q.dtype, dev)
    _check_tensor("k", k, q.dtype, dev)
    _check_tensor("w", w, torch.float32, dev, rows + (q.shape[-2],))
    _check_tensor("attn_softmax_l1norm", p, torch.float32, dev, rows + (n2, L))
    if metadata is not None:
        _check_tensor("metadata", metadata, torch.int32, dev, (METADATA_INTS,))
    if kl_loss is not None:
        _check_tensor("kl_loss", kl_loss, torch.float32, dev, rows + (n2,))
        desc.base.kl_loss = kl_loss.data_ptr()
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w), torch.empty_like(p))
    dq, dk, dw, y = out
    _check_tensor("dq", dq, q.dtype, dev, q.shape)
    _check_tensor("dk", dk, q.dtype, dev, k.shape)
    _check_tensor("dw", dw, torch.float32, dev, w.shape)
    _check_tensor("softmax_out", y, torch.float32, dev, p.shape)
    nbytes = _native.dense_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ms = _native.dense_grad_raw(desc, q.data_ptr(), k.data_ptr(), w.data_ptr(), p.data_ptr(),
                                metadata.data_ptr() if metadata is not None else 0, dq.data_ptr(),
                                dk.data_ptr(), dw.data_ptr(), y.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream_handle(dev),
                                profiled=profiled)
    return out, ms
