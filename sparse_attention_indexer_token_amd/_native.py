"""ctypes binding of libslikl.so (the C ABI declared in include/slikl.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels of the shared library.  If the library is missing the import of this
module still works, but every call raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libslikl.so")

SLIKL_OK = 0
SLIKL_ERR_NULLPTR = 1
SLIKL_ERR_PARAM_INVALID = 2
SLIKL_ERR_UNSUPPORTED = 3
SLIKL_ERR_WORKSPACE = 4
SLIKL_ERR_LAUNCH = 5

LAYOUT = {"BSND": 0, "TND": 1}
DTYPE = {"f16": 0, "bf16": 1}
SPLIT = {"weighted": 0, "rows": 1}
DK_MODE = {"auto": 0, "scatter": 1, "dense": 2, "sorted": 3}

METADATA_HEADER = 16
MAX_PARTS = 2048
METADATA_INTS = 2080
UNIT_OVERHEAD = 512
UNIT_OVERHEAD_DENSE = 1024

EXPORTS = ("slikl_grad_workspace_size", "slikl_grad_parts", "slikl_grad_unit_overhead", "slikl_grad_dk_strategy", "slikl_grad_metadata",
           "slikl_grad", "slikl_grad_profiled", "slikl_status_string", "slikl_grad_noalloc",
           "slikl_grad_noalloc_strategy", "slikl_attn_softmax_l1norm", "slikl_dense_grad_workspace_size",
           "slikl_dense_grad_metadata", "slikl_dense_grad", "slikl_dense_grad_profiled")
STATIC_SCRATCH_BYTES = 64 << 20

PHASES = ("metadata", "fill", "key_copy", "det_scale", "fused", "dk", "dk_final", "dk_prep", "dk_reduce")


class SliklDesc(ctypes.Structure):
    """Mirror of ``slikl_desc``."""
    _fields_ = [
        ("layout_q", c_int32), ("layout_k", c_int32), ("dtype", c_int32),
        ("deterministic", c_int32),
        ("batch", c_int64), ("s1", c_int64), ("s2", c_int64),
        ("n1", c_int64), ("n2", c_int64), ("d", c_int64), ("topk", c_int64),
        ("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p),
        ("num_parts", c_int32), ("split_mode", c_int32), ("dk_mode", c_int32),
        ("max_seqlen_q", c_int64), ("max_seqlen_k", c_int64),
        ("kl_loss", c_void_p),
        ("seq_used_q", c_void_p), ("seq_used_k", c_void_p),
    ]


class SliklDenseDesc(ctypes.Structure):
    """Mirror of ``slikl_dense_desc``."""
    _fields_ = [("base", SliklDesc), ("mask_mode", c_int32), ("cmp_ratio", c_int32)]


class SliklAttnPDesc(ctypes.Structure):
    """Mirror of ``slikl_attn_p_desc``."""
    _fields_ = [
        ("layout_q", c_int32), ("layout_k", c_int32), ("dtype", c_int32), ("reserved", c_int32),
        ("batch", c_int64), ("s1", c_int64), ("s2", c_int64),
        ("heads", c_int64), ("n2", c_int64), ("d", c_int64), ("topk", c_int64),
        ("scale", ctypes.c_float),
        ("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p),
    ]


class SliklError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


_lib = None


def load():
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_attention_indexer_token_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.slikl_grad_workspace_size.argtypes = [P(SliklDesc), P(c_size_t)]
    lib.slikl_grad_workspace_size.restype = c_int32
    lib.slikl_grad_parts.argtypes = [P(SliklDesc), P(c_int32)]
    lib.slikl_grad_parts.restype = c_int32
    lib.slikl_grad_unit_overhead.argtypes = [P(SliklDesc), P(c_int32)]
    lib.slikl_grad_unit_overhead.restype = c_int32
    lib.slikl_grad_dk_strategy.argtypes = [P(SliklDesc), P(c_int32)]
    lib.slikl_grad_dk_strategy.restype = c_int32
    lib.slikl_grad_metadata.argtypes = [P(SliklDesc), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.slikl_grad_metadata.restype = c_int32
    lib.slikl_grad.argtypes = [P(SliklDesc)] + [c_void_p] * 10 + [c_void_p, c_size_t, c_void_p]
    lib.slikl_grad.restype = c_int32
    lib.slikl_grad_profiled.argtypes = [P(SliklDesc)] + [c_void_p] * 10 + [c_void_p, c_size_t, c_void_p,
                                                                           P(ctypes.c_float)]
    lib.slikl_grad_profiled.restype = c_int32
    lib.slikl_grad_noalloc.argtypes = [P(SliklDesc)] + [c_void_p] * 10 + [c_void_p]
    lib.slikl_grad_noalloc.restype = c_int32
    lib.slikl_grad_noalloc_strategy.argtypes = [P(SliklDesc), P(c_int32)]
    lib.slikl_grad_noalloc_strategy.restype = c_int32
    lib.slikl_dense_grad_workspace_size.argtypes = [P(SliklDenseDesc), P(c_size_t)]
    lib.slikl_dense_grad_workspace_size.restype = c_int32
    lib.slikl_dense_grad_metadata.argtypes = [P(SliklDenseDesc), c_void_p, c_void_p, c_size_t, c_void_p]
    lib.slikl_dense_grad_metadata.restype = c_int32
    lib.slikl_dense_grad.argtypes = [P(SliklDenseDesc)] + [c_void_p] * 9 + [c_void_p, c_size_t, c_void_p]
    lib.slikl_dense_grad.restype = c_int32
    lib.slikl_dense_grad_profiled.argtypes = [P(SliklDenseDesc)] + [c_void_p] * 9 + [c_void_p, c_size_t, c_void_p,
                                                                                     P(ctypes.c_float)]
    lib.slikl_dense_grad_profiled.restype = c_int32
    lib.slikl_attn_softmax_l1norm.argtypes = [P(SliklAttnPDesc)] + [c_void_p] * 6
    lib.slikl_attn_softmax_l1norm.restype = c_int32
    lib.slikl_status_string.argtypes = [c_int32]
    lib.slikl_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().slikl_status_string(status).decode()
    except RuntimeError:
        return "library not loaded"


def _check(status: int, where: str):
    if status != SLIKL_OK:
        raise SliklError(status, where)


# ---------------------------------------------------------------------------
# Raw calls (pointers as ints).
# ---------------------------------------------------------------------------
def workspace_size(desc: SliklDesc) -> int:
    out = c_size_t(0)
    _check(load().slikl_grad_workspace_size(ctypes.byref(desc), ctypes.byref(out)),
           "slikl_grad_workspace_size")
    return out.value


def grad_parts(desc: SliklDesc) -> int:
    out = c_int32(0)
    _check(load().slikl_grad_parts(ctypes.byref(desc), ctypes.byref(out)), "slikl_grad_parts")
    return out.value


def unit_overhead(desc: SliklDesc) -> int:
    out = c_int32(0)
    _check(load().slikl_grad_unit_overhead(ctypes.byref(desc), ctypes.byref(out)), "slikl_grad_unit_overhead")
    return int(out.value)


def dk_strategy(desc: SliklDesc) -> str:
    out = c_int32(0)
    _check(load().slikl_grad_dk_strategy(ctypes.byref(desc), ctypes.byref(out)), "slikl_grad_dk_strategy")
    return {v: k for k, v in DK_MODE.items()}[int(out.value)]


def grad_metadata_raw(desc: SliklDesc, indices_ptr: int, metadata_ptr: int, ws_ptr: int,
                      ws_bytes: int, stream: int) -> None:
    _check(load().slikl_grad_metadata(ctypes.byref(desc), indices_ptr or None, metadata_ptr or None,
                                      ws_ptr or None, ws_bytes, stream or None),
           "slikl_grad_metadata")


def grad_raw(desc: SliklDesc, q, k, w, idx, p, metadata, dq, dk, dw, y, ws, ws_bytes, stream) -> None:
    _check(load().slikl_grad(ctypes.byref(desc), q or None, k or None, w or None, idx or None,
                             p or None, metadata or None, dq or None, dk or None, dw or None,
                             y or None, ws or None, ws_bytes, stream or None),
           "slikl_grad")


def grad_profiled_raw(desc: SliklDesc, q, k, w, idx, p, metadata, dq, dk, dw, y, ws, ws_bytes, stream) -> dict:
    ms = (ctypes.c_float * len(PHASES))()
    _check(load().slikl_grad_profiled(ctypes.byref(desc), q or None, k or None, w or None, idx or None,
                                      p or None, metadata or None, dq or None, dk or None, dw or None,
                                      y or None, ws or None, ws_bytes, stream or None, ms),
           "slikl_grad_profiled")
    return {name: float(ms[i]) for i, name in enumerate(PHASES)}


def noalloc_strategy(desc: SliklDesc) -> str:
    out = c_int32(0)
    _check(load().slikl_grad_noalloc_strategy(ctypes.byref(desc), ctypes.byref(out)),
           "slikl_grad_noalloc_strategy")
    return {v: k for k, v in DK_MODE.items()}[int(out.value)]


def grad_noalloc_raw(desc: SliklDesc, q, k, w, idx, p, metadata, dq, dk, dw, y, stream) -> None:
    _check(load().slikl_grad_noalloc(ctypes.byref(desc), q or None, k or None, w or None, idx or None,
                                     p or None, metadata or None, dq or None, dk or None, dw or None,
                                     y or None, stream or None),
           "slikl_grad_noalloc")


def attn_p_raw(desc: SliklAttnPDesc, q, k, idx, lse, p, stream) -> None:
    _check(load().slikl_attn_softmax_l1norm(ctypes.byref(desc), q or None, k or None, idx or None,
                                            lse or None, p or None, stream or None),
           "slikl_attn_softmax_l1norm")


def dense_workspace_size(desc: SliklDenseDesc) -> int:
    out = c_size_t(0)
    _check(load().slikl_dense_grad_workspace_size(ctypes.byref(desc), ctypes.byref(out)),
           "slikl_dense_grad_workspace_size")
    return out.value


def dense_metadata_raw(desc: SliklDenseDesc, metadata_ptr: int, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    _check(load().slikl_dense_grad_metadata(ctypes.byref(desc), metadata_ptr or None, ws_ptr or None, ws_bytes,
                                            stream or None), "slikl_dense_grad_metadata")


def dense_grad_raw(desc: SliklDenseDesc, q, k, w, p, metadata, dq, dk, dw, y, ws, ws_bytes, stream, profiled=False):
    args = (ctypes.byref(desc), q or None, k or None, w or None, p or None, metadata or None, dq or None,
            dk or None, dw or None, y or None, ws or None, ws_bytes, stream or None)
    if not profiled:
        _check(load().slikl_dense_grad(*args), "slikl_dense_grad")
        return None
    ms = (ctypes.c_float * len(PHASES))()
    _check(load().slikl_dense_grad_profiled(*args, ms), "slikl_dense_grad_profiled")
    return {name: float(ms[i]) for i, name in enumerate(PHASES)}
