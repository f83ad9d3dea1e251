"""C ABI checks that need no GPU: exported symbols and host-side validation.

slikl_grad_workspace_size touches no device, so every status path of the
descriptor validation is exercised here.  Compute entry points are only
called with descriptors that fail validation (they return before any HIP
call).
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_indexer_token_amd import _native
from sparse_attention_indexer_token_amd._native import SliklDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slikl.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        pytest.skip("libslikl.so not built")
    return _native.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(slikl_\w+)\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(_native.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for fn in header_functions():
        assert fn in names, fn
        assert getattr(lib, fn) is not None


def test_struct_layout_matches_header():
    # 4 x int32, 7 x int64, 2 pointers, 3 x int32 (+4 bytes of padding), 2 x int64
    assert ctypes.sizeof(SliklDesc) == 144
    assert SliklDesc.cu_seqlens_q.offset == 72
    assert SliklDesc.num_parts.offset == 88
    assert SliklDesc.dk_mode.offset == 96
    assert SliklDesc.max_seqlen_q.offset == 104
    assert SliklDesc.max_seqlen_k.offset == 112
    assert SliklDesc.kl_loss.offset == 120
    assert SliklDesc.seq_used_q.offset == 128
    assert SliklDesc.seq_used_k.offset == 136


def test_other_struct_layouts_match_header():
    # slikl_dense_desc: slikl_desc then two int32
    assert ctypes.sizeof(_native.SliklDenseDesc) == 152
    assert _native.SliklDenseDesc.mask_mode.offset == 144
    # slikl_attn_p_desc: 4 x int32, 7 x int64, float (+4 bytes of padding), 2 pointers
    assert ctypes.sizeof(_native.SliklAttnPDesc) == 96
    assert _native.SliklAttnPDesc.scale.offset == 72
    assert _native.SliklAttnPDesc.cu_seqlens_q.offset == 80


def good_desc(**kw):
    d = SliklDesc()
    d.layout_q = d.layout_k = 0
    d.dtype = 1
    d.deterministic = 0
    d.batch, d.s1, d.s2 = 1, 4096, 4096
    d.n1, d.n2, d.d, d.topk = 64, 1, 128, 2048
    d.cu_seqlens_q = d.cu_seqlens_k = None
    d.num_parts = 0
    d.split_mode = 0
    d.dk_mode = 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def ws(lib, d):
    n = ctypes.c_size_t(0)
    st = lib.slikl_grad_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_size_of_the_dsv32_shape(lib):
    st, n = ws(lib, good_desc(dk_mode=1))
    assert st == 0
    acc = 4096 * 1 * 128 * 4
    assert n >= acc + 2080 * 4 + (4096 + 1) * 8
    st, n_det = ws(lib, good_desc(deterministic=1, dk_mode=1))
    assert st == 0 and n_det >= n + 4096 * 128 * 4
    # dense records: dI and 64 head bits per (row, key) dominate
    st, n_dense = ws(lib, good_desc())
    assert st == 0 and n_dense >= 4096 * 4096 * (4 + 8)


def tnd_desc(cu, **kw):
    d = good_desc(layout_q=1, layout_k=1, **kw)
    d.cu_seqlens_q = ctypes.cast(cu, ctypes.c_void_p)
    d.cu_seqlens_k = ctypes.cast(cu, ctypes.c_void_p)
    return d


def test_dense_mode_with_tnd_needs_the_maxima(lib):
    cu = (ctypes.c_int32 * 2)(0, 4096)
    assert ws(lib, tnd_desc(cu, dk_mode=2))[0] == 3                        # no maxima given
    assert ws(lib, tnd_desc(cu, dk_mode=2, max_seqlen_q=4096))[0] == 3     # only one side
    st, n = ws(lib, tnd_desc(cu, dk_mode=2, max_seqlen_q=4096, max_seqlen_k=4096))
    st_b, n_b = ws(lib, good_desc(dk_mode=2))
    # the same records as the BSND problem, plus one int4 of row info per query row
    assert st == 0 and st_b == 0 and n >= n_b and n - n_b <= 4096 * 16 + 1024
    assert ws(lib, tnd_desc(cu, max_seqlen_q=-1))[0] == 2
    assert ws(lib, tnd_desc(cu, max_seqlen_k=1 << 31))[0] == 2
    # BSND sides ignore the fields
    assert ws(lib, good_desc(max_seqlen_q=-5, max_seqlen_k=-5))[0] == 0


@pytest.mark.parametrize("field,value,status", [
    ("layout_q", 2, 2), ("layout_k", -1, 2), ("dtype", 5, 2), ("deterministic", 2, 2),
    ("batch", 0, 2), ("s1", 0, 2), ("s2", 0, 2), ("n1", 0, 2), ("n1", 129, 2),
    ("n2", 3, 2), ("n2", 0, 2), ("d", 96, 2), ("d", 256, 2), ("topk", 0, 2), ("topk", 2049, 2),
    ("num_parts", 2049, 2), ("num_parts", -1, 2), ("split_mode", 2, 2), ("dk_mode", 4, 2),
    ("layout_q", 1, 1),                      # TND q without cu_seqlens_q
    ("layout_k", 1, 1),                      # TND k without cu_seqlens_k
    ("s1", 1 << 40, 2),                      # more than 2^31 elements
])
def test_validation_status(lib, field, value, status):
    st, _ = ws(lib, good_desc(**{field: value}))
    assert st == status


def test_tnd_total_may_be_zero(lib):
    cu = (ctypes.c_int32 * 2)(0, 0)
    d = good_desc(layout_q=1, layout_k=1, s1=0, s2=0)
    d.cu_seqlens_q = ctypes.cast(cu, ctypes.c_void_p)
    d.cu_seqlens_k = ctypes.cast(cu, ctypes.c_void_p)
    st, n = ws(lib, d)
    assert st == 0 and n > 0


def test_null_pointers(lib):
    n = ctypes.c_size_t(0)
    assert lib.slikl_grad_workspace_size(None, ctypes.byref(n)) == 1
    d = good_desc()
    assert lib.slikl_grad_workspace_size(ctypes.byref(d), None) == 1
    # execute entry points: null tensors fail before any device work
    assert lib.slikl_grad(ctypes.byref(d), *([None] * 10), None, 0, None) == 1
    assert lib.slikl_grad_metadata(ctypes.byref(d), None, None, None, 0, None) == 1
    assert lib.slikl_grad_profiled(ctypes.byref(d), *([None] * 10), None, 0, None, None) == 1


def test_unit_overhead_follows_the_dk_strategy(lib):
    def oh(d):
        out = ctypes.c_int32(-1)
        st = lib.slikl_grad_unit_overhead(ctypes.byref(d), ctypes.byref(out))
        return st, out.value
    # auto mode: dense when S2 <= 16 topk (32 topk when deterministic), BSND, records fit
    assert oh(good_desc()) == (0, _native.UNIT_OVERHEAD_DENSE)             # dsv32 shape
    assert oh(good_desc(dk_mode=2)) == (0, _native.UNIT_OVERHEAD_DENSE)
    assert oh(good_desc(dk_mode=1)) == (0, _native.UNIT_OVERHEAD)
    assert oh(good_desc(topk=256)) == (0, _native.UNIT_OVERHEAD_DENSE)     # S2 = 16 topk
    assert oh(good_desc(topk=128)) == (0, _native.UNIT_OVERHEAD_DENSE)     # sparser lists: sorted
    assert oh(good_desc(topk=128, dk_mode=1)) == (0, _native.UNIT_OVERHEAD)
    assert oh(good_desc(topk=128, n1=128)) == (0, _native.UNIT_OVERHEAD_DENSE)   # sorted
    assert oh(good_desc(topk=128, n1=128, dk_mode=1)) == (0, _native.UNIT_OVERHEAD)
    assert oh(good_desc(topk=128, deterministic=1)) == (0, _native.UNIT_OVERHEAD_DENSE)
    assert oh(good_desc(topk=64, deterministic=1)) == (0, _native.UNIT_OVERHEAD_DENSE)  # sorted
    cu = (ctypes.c_int32 * 2)(0, 4096)
    assert oh(tnd_desc(cu)) == (0, _native.UNIT_OVERHEAD_DENSE)           # TND without maxima: sorted
    assert oh(tnd_desc(cu, max_seqlen_q=4096, max_seqlen_k=4096)) == (0, _native.UNIT_OVERHEAD_DENSE)
    assert oh(tnd_desc(cu, max_seqlen_q=4096, max_seqlen_k=65536)) == (0, _native.UNIT_OVERHEAD_DENSE)
    assert oh(good_desc(d=96))[0] == 2
    out = ctypes.c_int32(0)
    assert lib.slikl_grad_unit_overhead(None, ctypes.byref(out)) == 1
    assert lib.slikl_grad_unit_overhead(ctypes.byref(good_desc()), None) == 1


def test_dk_strategy_query_resolves_auto(lib):
    def strat(d):
        out = ctypes.c_int32(-1)
        st = lib.slikl_grad_dk_strategy(ctypes.byref(d), ctypes.byref(out))
        return st, out.value
    assert strat(good_desc()) == (0, 2)                        # dsv32 shape: dense
    assert strat(good_desc(topk=128)) == (0, 3)                # S2 > 16 topk: sorted
    assert strat(good_desc(topk=128, n1=128)) == (0, 3)        # 128-head groups: sorted too
    assert strat(good_desc(topk=128, s1=1024)) == (0, 1)       # under 2048 units: scatter
    assert strat(good_desc(topk=128, deterministic=1)) == (0, 2)   # S2 <= 32 topk
    assert strat(good_desc(dk_mode=1)) == (0, 1)
    assert strat(good_desc(dk_mode=3)) == (0, 3)
    assert strat(good_desc(dk_mode=3, deterministic=1)) == (0, 3)
    assert strat(good_desc(dk_mode=3, n1=128)) == (0, 3)
    assert strat(good_desc(dk_mode=3, n1=128, n2=2)) == (0, 3)
    # head groups up to 64 run the 64-head kernel: N2 * D * 2 below 16384 bytes
    assert strat(good_desc(dk_mode=3, n1=64, n2=64, d=128, s2=512))[0] == 3
    assert strat(good_desc(dk_mode=3, n1=64, n2=32, d=128, s2=512)) == (0, 3)
    # 32-bit record indices: T1 * N2 * topk below 2^31 - 65536
    assert strat(good_desc(dk_mode=3, s1=1048576 - 33, topk=2048, n1=1, d=32, s2=64))[0] == 0
    assert strat(good_desc(dk_mode=3, s1=1048576 - 32, topk=2048, n1=1, d=32, s2=64))[0] == 3
    cu = (ctypes.c_int32 * 2)(0, 4096)
    assert strat(tnd_desc(cu, dk_mode=3)) == (0, 3)            # no maxima needed
    assert strat(tnd_desc(cu)) == (0, 3)                       # no maxima: not dense
    assert strat(tnd_desc(cu, dk_mode=1)) == (0, 1)
    assert lib.slikl_grad_dk_strategy(None, ctypes.byref(ctypes.c_int32(0))) == 1
    assert lib.slikl_grad_dk_strategy(ctypes.byref(good_desc()), None) == 1


def test_sorted_mode_workspace_holds_the_parts(lib):
    st, n_sc = ws(lib, good_desc(dk_mode=1))
    st2, n_so = ws(lib, good_desc(dk_mode=3))
    assert st == 0 and st2 == 0
    slots = 4096 * 2048
    # rows of D (sized for fp32, the format taken when a key takes many parts), sort
    # pairs and list
    assert n_so - n_sc >= slots * (128 * 4 + 12)


def test_small_workspace_is_rejected_before_launch(lib):
    d = good_desc(num_parts=4)
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
    st = lib.slikl_grad(ctypes.byref(d), *([fake] * 10), fake, 16, None)
    assert st == 4
    st = lib.slikl_grad_metadata(ctypes.byref(d), fake, fake, fake, 16, None)
    assert st == 4


def test_status_strings(lib):
    for s in range(6):
        assert lib.slikl_status_string(s)
    assert b"unknown" in lib.slikl_status_string(99)


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"^#define (SLIKL_\w+) (\d+)", text, flags=re.M))
    assert int(defs["SLIKL_METADATA_HEADER"]) == _native.METADATA_HEADER
    assert int(defs["SLIKL_MAX_PARTS"]) == _native.MAX_PARTS
    assert int(defs["SLIKL_METADATA_INTS"]) == _native.METADATA_INTS
    assert int(defs["SLIKL_UNIT_OVERHEAD"]) == _native.UNIT_OVERHEAD
    assert int(defs["SLIKL_UNIT_OVERHEAD_DENSE"]) == _native.UNIT_OVERHEAD_DENSE


def test_seq_used_applies_to_tnd_sides_only():
    import torch
    import sparse_attention_indexer_token_amd as slikl
    q = torch.zeros(1, 8, 4, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    idx = torch.zeros(1, 8, 1, 4, dtype=torch.int32)
    used = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        slikl.make_desc(q, k, idx, seq_used_q=used)          # BSND query side
    with pytest.raises(ValueError):
        slikl.make_desc(q, k, idx, seq_used_k=used)          # BSND key side
    d = slikl.make_desc(q, k, idx)
    assert d.seq_used_q is None and d.seq_used_k is None and d.kl_loss is None


def test_optional_outputs_do_not_change_the_workspace(lib):
    base = ws(lib, good_desc())
    d = good_desc()
    d.kl_loss = 0x1000                  # never dereferenced by the size query
    assert ws(lib, d) == base
