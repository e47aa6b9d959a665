"""The C-ABI library on the CPU: it loads, exports every declared symbol, its
host-only results match the oracle bit for bit, and every invalid argument is
rejected before any GPU work.  No kernel is launched here."""

import ctypes
import os
import re
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import workloads
import structured_sparse_head_amd as fa
from structured_sparse_head_amd import fibatt as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "fibatt.h")) as fh:
        text = fh.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(fibatt_\w+)\s*\(", text, re.M))
    assert declared == set(fa.EXPORTED)
    L = fa.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_wythoff_matches_oracle():
    for i in range(1, 1001):
        assert fa.wythoff(i) == oracle.wythoff_row(i), i


def test_wythoff_large_rows_match_decimal_closed_form():
    getcontext().prec = 80
    phi = (Decimal(1) + Decimal(5).sqrt()) / 2
    rng = np.random.default_rng(5)
    rows = [int(x) for x in rng.integers(1000, 800_000_000, size=300)] + [820_000_000]
    for i in rows:
        p = int((Decimal(i) * phi).to_integral_value(rounding="ROUND_FLOOR"))
        a = int((Decimal(p) * phi).to_integral_value(rounding="ROUND_FLOOR"))
        b = int((Decimal(p) * phi * phi).to_integral_value(rounding="ROUND_FLOOR"))
        if b > 2 ** 31 - 1:
            with pytest.raises(fa.FibattError) as ei:
                fa.wythoff(i)
            assert ei.value.code == fa.E_RANGE
        else:
            assert fa.wythoff(i) == (a, b), i


def test_wythoff_modified_matches_oracle():
    for i in range(1, 1001):
        assert fa.wythoff_modified(i) == oracle.wythoff_row_modified(i), i
    a, b = fa.wythoff_rows(12, modified=True)
    oa, ob = oracle.wythoff_rows(12, modified=True)
    assert np.array_equal(a, oa) and np.array_equal(b, ob)


def test_wythoff_rows_near_the_int32_limit():
    # Rows whose floor(i phi) needs more than 64 bits in 5 n^2 (n ~ 1.9e9 and
    # up): the modified pair (i - 1, floor(i phi)) still fits int32 below
    # i = 1,327,217,885, the plain row does not.
    getcontext().prec = 80
    phi = (Decimal(1) + Decimal(5).sqrt()) / 2
    for i in (1_200_000_000, 1_300_000_000, 1_327_217_884, 1_327_217_885, 2 ** 31 - 1):
        p = int((Decimal(i) * phi).to_integral_value(rounding="ROUND_FLOOR"))
        if p <= 2 ** 31 - 1:
            assert fa.wythoff_modified(i) == (i - 1, p), i
        else:
            with pytest.raises(fa.FibattError) as ei:
                fa.wythoff_modified(i)
            assert ei.value.code == fa.E_RANGE
        with pytest.raises(fa.FibattError) as ei:  # a = floor(p phi) > 2^31 - 1
            fa.wythoff(i)
        assert ei.value.code == fa.E_RANGE
    assert fa.wythoff_modified(1_200_000_000) == (1_199_999_999, 1_941_640_786)


def test_wythoff_modified_rejects_bad_rows():
    for i in (0, -5):
        with pytest.raises(fa.FibattError) as ei:
            fa.wythoff_modified(i)
        assert ei.value.code == fa.E_INVAL


def test_windows_match_oracle():
    for H in (1, 2, 3, 12, 16, 100):
        for w_min, w_max in ((1, 1), (5, 65), (49, 197), (1, 2 ** 31 - 1), (7, 8)):
            assert list(fa.windows(H, w_min, w_max)) == oracle.window_sizes(H, w_min, w_max)
    for H, lo, hi in ((0, 1, 2), (3, 0, 2), (3, 5, 4)):
        with pytest.raises(fa.FibattError) as ei:
            fa.windows(H, lo, hi)
        assert ei.value.code == fa.E_INVAL


def test_wythoff_rejects_bad_rows():
    for i in (0, -1, -(2 ** 31)):
        with pytest.raises(fa.FibattError) as ei:
            fa.wythoff(i)
        assert ei.value.code == fa.E_INVAL


@pytest.mark.parametrize("num", sorted(workloads.WORKLOADS))
def test_offset_tables_bit_exact_for_workloads(num):
    wl = workloads.WORKLOADS[num]
    a, b = oracle.wythoff_rows(wl.H)
    w = workloads.windows(wl)
    ptr, offs = fa.offsets(wl.N, a, b, w)
    optr, ooffs = oracle.offset_table(wl.N, a, b, w)
    assert np.array_equal(ptr, optr)
    assert np.array_equal(offs, ooffs)


def test_offset_tables_bit_exact_random():
    rng = np.random.default_rng(11)
    for _ in range(400):
        H = int(rng.integers(1, 20))
        N = int(rng.choice([1, 2, 3, 5, 17, 100, 1000, 70000, 2 ** 31 - 1]))
        a = rng.integers(0, 60, size=H)
        b = rng.integers(1, 60, size=H)
        w = rng.integers(1, min(N, 10 ** 9) + 1, size=H)
        if rng.random() < 0.3:
            a[:] = rng.integers(0, 3, size=H)
            b[:] = rng.integers(1, 3, size=H)
        ptr, offs = fa.offsets(N, a, b, w)
        optr, ooffs = oracle.offset_table(N, a, b, w)
        assert np.array_equal(ptr, optr), (N, a, b, w)
        assert np.array_equal(offs, ooffs), (N, a, b, w)


def test_offsets_two_call_sizing_and_errors():
    L = fa.lib()
    a, b, w = fb._i32([1, 4]), fb._i32([2, 7]), fb._i32([197, 197])
    ptr = np.zeros(3, dtype=np.int32)
    rc = L.fibatt_offsets(2, 197, fb._ptr(a), fb._ptr(b), fb._ptr(w), fb._ptr(ptr), None, 0)
    assert rc == fa.E_RANGE and list(ptr) == [0, 11, 19]
    small = np.zeros(5, dtype=np.int32)
    rc = L.fibatt_offsets(2, 197, fb._ptr(a), fb._ptr(b), fb._ptr(w), fb._ptr(ptr),
                          fb._ptr(small), 5)
    assert rc == fa.E_RANGE and ptr[-1] == 19
    assert b"capacity" in L.fibatt_last_error()
    bad = [
        (0, 197, a, b, w), (2, 0, a, b, w),
        (2, 197, fb._i32([-1, 4]), b, w), (2, 197, a, fb._i32([2, 0]), w),
        (2, 197, a, b, fb._i32([0, 197])), (2, 197, a, b, fb._i32([197, 198])),
    ]
    for H, N, aa, bb, ww in bad:
        rc = L.fibatt_offsets(H, N, fb._ptr(aa), fb._ptr(bb), fb._ptr(ww), fb._ptr(ptr), None, 0)
        assert rc == fa.E_INVAL, (H, N)
        assert L.fibatt_last_error() != b""
    rc = L.fibatt_offsets(2, 197, None, fb._ptr(b), fb._ptr(w), fb._ptr(ptr), None, 0)
    assert rc == fa.E_INVAL
    rc = L.fibatt_offsets(2, 197, fb._ptr(a), fb._ptr(b), fb._ptr(w), None, None, 0)
    assert rc == fa.E_INVAL


# --------------------------------------------------------------------------
# fwd / bwd argument validation (fails before any launch, so no GPU needed)
# --------------------------------------------------------------------------

class _Case:
    def __init__(self, **kw):
        p = dict(B=2, H=3, N=65, d_h=64, dtype=fa.BF16, a=[1, 4, 6], b=[2, 7, 10],
                 w=[65, 65, 65])
        p.update(kw)
        self.a, self.b, self.w = fb._i32(p["a"]), fb._i32(p["b"]), fb._i32(p["w"])
        self.desc = fb.Desc(p["B"], p["H"], p["N"], p["d_h"], p["dtype"],
                            fb._ptr(self.a), fb._ptr(self.b), fb._ptr(self.w))


GOOD = 0x10000  # aligned dummy address, never dereferenced on these paths


def _fwd(desc, q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD):
    return fa.lib().fibatt_fwd(ctypes.byref(desc) if desc is not None else None, q, k, v, o, lse,
                               None)


def _bwd(desc, ptrs=None):
    p = [GOOD] * 9 if ptrs is None else ptrs
    return fa.lib().fibatt_bwd(ctypes.byref(desc) if desc is not None else None, *p, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), fa.E_INVAL), (dict(H=0, a=[], b=[], w=[]), fa.E_INVAL), (dict(N=0), fa.E_INVAL),
    (dict(d_h=32), fa.E_UNSUPPORTED), (dict(d_h=96), fa.E_UNSUPPORTED),
    (dict(dtype=7), fa.E_UNSUPPORTED),
    (dict(H=129, a=[1] * 129, b=[2] * 129, w=[65] * 129), fa.E_UNSUPPORTED),
    (dict(a=[-1, 4, 6]), fa.E_INVAL), (dict(b=[2, 0, 10]), fa.E_INVAL),
    (dict(a=[0, 4, 6], b=[0, 7, 10]), fa.E_INVAL),
    (dict(w=[65, 0, 65]), fa.E_INVAL), (dict(w=[65, 66, 65]), fa.E_INVAL),
])
def test_fwd_bwd_reject_bad_descriptors(kw, code):
    c = _Case(**kw)
    assert _fwd(c.desc) == code
    assert fa.lib().fibatt_last_error() != b""
    assert _bwd(c.desc) == code
    assert fa.lib().fibatt_bwd_workspace_floats(ctypes.byref(c.desc)) == -1


def test_fwd_bwd_reject_null_and_misaligned_pointers():
    c = _Case()
    assert _fwd(None) == fa.E_INVAL
    for i in range(5):
        args = [GOOD] * 5
        args[i] = None
        assert _fwd(c.desc, *args) == fa.E_INVAL
        args[i] = GOOD + 4
        assert _fwd(c.desc, *args) == fa.E_INVAL
        assert b"aligned" in fa.lib().fibatt_last_error()
    assert _bwd(None) == fa.E_INVAL
    for i in range(9):
        ptrs = [GOOD] * 9
        ptrs[i] = None
        assert _bwd(c.desc, ptrs) == fa.E_INVAL
        ptrs[i] = GOOD + 8
        assert _bwd(c.desc, ptrs) == fa.E_INVAL


def test_null_head_arrays_rejected():
    c = _Case()
    c.desc.a = ctypes.POINTER(ctypes.c_int32)()
    assert _fwd(c.desc) == fa.E_INVAL
    assert _bwd(c.desc) == fa.E_INVAL


def test_workspace_size():
    c = _Case()
    assert fa.lib().fibatt_bwd_workspace_floats(ctypes.byref(c.desc)) == 2 * 3 * 65


def test_binding_refuses_host_tensors():
    import torch
    op = fa.Fibottention(2, 3, 65, 64, torch.float32, [1, 4, 6], [2, 7, 10], [65] * 3)
    q = torch.zeros(2, 3, 65, 64)
    with pytest.raises(ValueError):
        op.forward(q, q, q, o=q, lse=torch.zeros(2, 3, 65))
    # strided views of host memory are refused too, before any library call
    qkv = torch.zeros(2, 65, 3, 3, 64)
    v = qkv[:, :, 0].permute(0, 2, 1, 3)
    assert not v.is_contiguous()
    with pytest.raises(ValueError):
        op.forward(v, v, v, o=q, lse=torch.zeros(2, 3, 65))
    with pytest.raises(ValueError):
        op.backward(v, v, v, torch.zeros(2, 3, 65), v, dq=q, dk=q, dv=q,
                    workspace=torch.zeros(2 * 3 * 65))


def test_qkv_function_rejects_bad_layouts():
    import torch
    with pytest.raises(ValueError):
        fa.FibottentionQKVFunction.apply(torch.zeros(2, 65, 2, 3, 64), [1, 4, 6], [2, 7, 10],
                                         [65] * 3, False)
    with pytest.raises(ValueError):   # not contiguous
        fa.FibottentionQKVFunction.apply(torch.zeros(2, 3, 65, 3, 64).transpose(1, 2),
                                         [1, 4, 6], [2, 7, 10], [65] * 3, False)


# --------------------------------------------------------------------------
# Class-token entry points: validation and workspace sizes (no launch)
# --------------------------------------------------------------------------

def _fwd_cls(desc, q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD, ws=GOOD):
    return fa.lib().fibatt_fwd_cls(ctypes.byref(desc) if desc is not None else None, q, k, v, o,
                                   lse, ws, None)


def _bwd_cls(desc, ptrs=None):
    p = [GOOD] * 9 if ptrs is None else ptrs
    return fa.lib().fibatt_bwd_cls(ctypes.byref(desc) if desc is not None else None, *p, None)


def test_cls_entry_points_reject_bad_arguments():
    bad = _Case(w=[65, 66, 65])
    assert _fwd_cls(bad.desc) == fa.E_INVAL
    assert _bwd_cls(bad.desc) == fa.E_INVAL
    assert fa.lib().fibatt_fwd_cls_workspace_floats(ctypes.byref(bad.desc)) == -1
    assert fa.lib().fibatt_bwd_cls_workspace_floats(ctypes.byref(bad.desc)) == -1
    c = _Case()
    assert _fwd_cls(None) == fa.E_INVAL
    for i in range(5):
        args = [GOOD] * 6
        args[i] = None
        assert _fwd_cls(c.desc, *args) == fa.E_INVAL
        args[i] = GOOD + 4
        assert _fwd_cls(c.desc, *args) == fa.E_INVAL
    for i in range(9):
        ptrs = [GOOD] * 9
        ptrs[i] = None
        assert _bwd_cls(c.desc, ptrs) == fa.E_INVAL
    # N > 1024 needs a forward workspace; a NULL one is rejected
    big = _Case(N=2049, w=[2049] * 3)
    assert _fwd_cls(big.desc, ws=None) == fa.E_INVAL
    assert b"workspace" in fa.lib().fibatt_last_error()


def test_cls_workspace_sizes():
    c = _Case()   # B=2, H=3, N=65, d_h=64: one range per slab
    assert fa.lib().fibatt_fwd_cls_workspace_floats(ctypes.byref(c.desc)) == 0
    assert fa.lib().fibatt_bwd_cls_workspace_floats(ctypes.byref(c.desc)) == 2 * 3 * (65 + 64) + 64
    big = _Case(N=2049, w=[2049] * 3, d_h=128)   # three ranges of 1024 rows
    assert fa.lib().fibatt_fwd_cls_workspace_floats(ctypes.byref(big.desc)) == 6 * 3 * 130
    assert fa.lib().fibatt_bwd_cls_workspace_floats(ctypes.byref(big.desc)) == \
        6 * (2049 + 128) + 128 + 6 * 3 * 257


# --------------------------------------------------------------------------
# Distance-table heads: validation and workspace sizes (no launch)
# --------------------------------------------------------------------------

def _tdesc(ptr, offs, B=2, H=None, N=65, d_h=64, dtype=fa.BF16, cls=0, dev=GOOD):
    ptr, offs = fb._i32(ptr), fb._i32(offs)
    H = len(ptr) - 1 if H is None else H
    d = fb.TableDesc(B, H, N, d_h, dtype, cls, fb._ptr(ptr), fb._ptr(offs), dev)
    d._keep = (ptr, offs)
    return d


def _fwd_t(d, ws=GOOD):
    return fa.lib().fibatt_fwd_table(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, ws, None)


def test_table_validation():
    L = fa.lib()
    good = _tdesc([0, 3, 3, 5], [1, 2, 4, 0, 7])
    assert L.fibatt_bwd_table_workspace_floats(ctypes.byref(good)) == 2 * 3 * 65
    assert L.fibatt_fwd_table_workspace_floats(ctypes.byref(good)) == 0
    cases = [
        (_tdesc([1, 3], [1, 2, 3]), fa.E_INVAL, b"head_ptr[0]"),
        (_tdesc([0, 3, 2], [1, 2, 3]), fa.E_INVAL, b"non-decreasing"),
        (_tdesc([0, 3], [1, 3, 2]), fa.E_INVAL, b"ascending"),
        (_tdesc([0, 2], [1, 1]), fa.E_INVAL, b"ascending"),
        (_tdesc([0, 2], [-1, 3]), fa.E_INVAL, b"outside"),
        (_tdesc([0, 2], [1, 65]), fa.E_INVAL, b"outside"),
        (_tdesc([0, 65], list(range(65)), N=100), fa.E_UNSUPPORTED, b"at most 64"),
        (_tdesc([0, 2], [1, 2], cls=2), fa.E_INVAL, b"cls"),
        (_tdesc([0, 2], [1, 2], dev=None), fa.E_INVAL, b"offs_device"),
        (_tdesc([0, 2], [1, 2], dev=GOOD + 2), fa.E_INVAL, b"aligned"),
        (_tdesc([0, 2], [1, 2], d_h=96), fa.E_UNSUPPORTED, b"d_h"),
    ]
    for d, code, msg in cases:
        assert _fwd_t(d) == code, msg
        assert msg in L.fibatt_last_error(), (msg, L.fibatt_last_error())
        assert L.fibatt_bwd_table_workspace_floats(ctypes.byref(d)) == -1
    # an empty table is valid (every row empty) and needs no device copy
    assert L.fibatt_bwd_table_workspace_floats(ctypes.byref(_tdesc([0, 0], [], dev=None))) \
        == 2 * 65
    # class-token mask: workspace as for fibatt_*_cls
    big = _tdesc([0, 2], [1, 2], N=2049, d_h=128, cls=1)
    assert L.fibatt_fwd_table_workspace_floats(ctypes.byref(big)) == 2 * 3 * 130
    assert _fwd_t(big, ws=None) == fa.E_INVAL


def test_table_binding_checks_shapes():
    import torch
    op = fa.FibottentionTable.__new__(fa.FibottentionTable)
    op.shape, op.dtype = (2, 3, 65, 64), torch.float32
    op._offs_dev = torch.zeros(1, dtype=torch.int32)  # a CPU stand-in for the device copy
    with pytest.raises(ValueError):
        op._shapes(torch.zeros(2, 3, 64, 64))
    with pytest.raises(ValueError):
        op._shapes(torch.zeros(2, 3, 65, 64, dtype=torch.bfloat16))
    op._shapes(torch.zeros(2, 3, 65, 64))  # matching shape, dtype and device


# --------------------------------------------------------------------------
# Strided entry points: layout validation (no launch)
# --------------------------------------------------------------------------

def _dense_layouts(B=2, H=3, N=65, d=64):
    ls = fb.Layouts()
    for name, _ in fb.Layouts._fields_:
        setattr(ls, name, fb.Layout(H * N * d, N * d, d))
    return ls


def _fwd_s(desc, ls, cls=0, ptrs=None):
    p = [GOOD] * 6 if ptrs is None else ptrs
    return fa.lib().fibatt_fwd_strided(ctypes.byref(desc), cls,
                                       ctypes.byref(ls) if ls is not None else None, *p, None)


def _bwd_s(desc, ls, cls=0, ptrs=None):
    p = [GOOD] * 9 if ptrs is None else ptrs
    return fa.lib().fibatt_bwd_strided(ctypes.byref(desc), cls,
                                       ctypes.byref(ls) if ls is not None else None, *p, None)


@pytest.mark.parametrize("field,layout,msg", [
    ("q", (-64, 64, 64), b"strides must be >= 0"),
    ("k", (0, 0, 32), b"sn = 32 must be >= d_h"),
    ("v", (4, 64, 64), b"multiples of 8"),      # bf16: 16 bytes = 8 elements
    ("o", ((1 << 62) - 8, 64, 64), b"2^62"),
])
def test_strided_forward_rejects_bad_layouts(field, layout, msg):
    c = _Case()
    ls = _dense_layouts()
    setattr(ls, field, fb.Layout(*layout))
    assert _fwd_s(c.desc, ls) == fa.E_INVAL
    assert msg in fa.lib().fibatt_last_error()


@pytest.mark.parametrize("field,layout,msg", [
    ("dout", (8, 64, 63), b"sn = 63"),
    ("dq", (2, 64, 64), b"multiples of 4"),      # fp32 gradients: 4 elements
    ("dk", (0, -1, 64), b">= 0"),
    ("dv", (0, 1 << 60, 1 << 60), b"2^62"),
])
def test_strided_backward_rejects_bad_layouts(field, layout, msg):
    c = _Case()
    ls = _dense_layouts()
    setattr(ls, field, fb.Layout(*layout))
    assert _bwd_s(c.desc, ls) == fa.E_INVAL
    assert msg in fa.lib().fibatt_last_error()


@pytest.mark.parametrize("field,layout", [
    ("o", (0, 65 * 64, 64)),        # B = 2 slabs of a batch would share rows
    ("o", (3 * 65 * 64, 0, 64)),    # H = 3 heads would share rows
])
def test_strided_forward_rejects_broadcast_outputs(field, layout):
    c = _Case()
    ls = _dense_layouts()
    setattr(ls, field, fb.Layout(*layout))
    assert _fwd_s(c.desc, ls) == fa.E_INVAL
    assert b"broadcast strides are for inputs only" in fa.lib().fibatt_last_error()


@pytest.mark.parametrize("field,layout", [
    ("dq", (0, 65 * 64, 64)),
    ("dk", (3 * 65 * 64, 0, 64)),
    ("dv", (0, 0, 64)),
])
def test_strided_backward_rejects_broadcast_outputs(field, layout):
    c = _Case()
    ls = _dense_layouts()
    setattr(ls, field, fb.Layout(*layout))
    assert _bwd_s(c.desc, ls) == fa.E_INVAL
    assert b"broadcast strides are for inputs only" in fa.lib().fibatt_last_error()


def test_strided_zero_strides_allowed_where_nothing_is_shared():
    # Inputs may broadcast; an output may have a zero stride along an axis of
    # extent 1.  Both then pass the layout checks and stop at a NULL pointer.
    c = _Case()
    ls = _with(_dense_layouts(), q=fb.Layout(0, 0, 64), k=fb.Layout(0, 65 * 64, 64))
    assert _fwd_s(c.desc, ls, ptrs=[GOOD] * 4 + [None, GOOD]) == fa.E_INVAL
    assert b"lse is NULL" in fa.lib().fibatt_last_error()
    one = _Case(B=1)
    ls1 = _with(_dense_layouts(B=1), o=fb.Layout(0, 65 * 64, 64))
    assert _fwd_s(one.desc, ls1, ptrs=[GOOD] * 4 + [None, GOOD]) == fa.E_INVAL
    assert b"lse is NULL" in fa.lib().fibatt_last_error()


def test_strided_layouts_of_unused_tensors_are_ignored():
    c = _Case(dtype=fa.F32)
    ls = _dense_layouts()
    ls.o = fb.Layout(-1, -1, -1)       # the backward does not read o
    ls.dq = fb.Layout(-1, -1, -1)      # the forward does not read dq, dk, dv, dout
    ls.dout = fb.Layout(-1, -1, -1)
    # both then fail on a later check (a NULL pointer), not on the layouts
    assert _fwd_s(c.desc, _with(ls, o=fb.Layout(3 * 65 * 64, 65 * 64, 64)),
                  ptrs=[GOOD, GOOD, GOOD, GOOD, None, GOOD]) == fa.E_INVAL
    assert b"lse is NULL" in fa.lib().fibatt_last_error()
    ls2 = _with(_dense_layouts(), o=fb.Layout(-1, -1, -1))
    assert _bwd_s(c.desc, ls2, ptrs=[GOOD] * 8 + [None]) == fa.E_INVAL
    assert b"workspace is NULL" in fa.lib().fibatt_last_error()


def _with(ls, **kw):
    out = fb.Layouts()
    for name, _ in fb.Layouts._fields_:
        setattr(out, name, kw.get(name, getattr(ls, name)))
    return out


def test_strided_entry_points_reject_bad_arguments():
    c = _Case()
    ls = _dense_layouts()
    assert _fwd_s(c.desc, None) == fa.E_INVAL
    assert _bwd_s(c.desc, None) == fa.E_INVAL
    assert _fwd_s(c.desc, ls, cls=2) == fa.E_INVAL
    assert _bwd_s(c.desc, ls, cls=-1) == fa.E_INVAL
    for i in range(5):
        p = [GOOD] * 6
        p[i] = GOOD + 4
        assert _fwd_s(c.desc, ls, ptrs=p) == fa.E_INVAL
        assert b"aligned" in fa.lib().fibatt_last_error()
    bad = _Case(w=[65, 66, 65])
    assert _fwd_s(bad.desc, ls) == fa.E_INVAL


def test_measurement_aids_reject_bad_arguments():
    L = fa.lib()
    fake = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first
    arr = (ctypes.c_void_p * 1)(fake.value)
    # fibatt_hbm_stream
    assert L.fibatt_hbm_stream(arr, 0, arr, 1, 1024, 1, None) == fb.E_INVAL
    assert L.fibatt_hbm_stream(arr, 1, arr, 5, 1024, 1, None) == fb.E_INVAL
    assert L.fibatt_hbm_stream(arr, 1, arr, 1, 1024, 3, None) == fb.E_INVAL
    assert L.fibatt_hbm_stream(arr, 1, arr, 1, 1000, 1, None) == fb.E_INVAL
    assert "multiple of 16" in L.fibatt_last_error().decode()
    # fibatt_fabric_read
    mib4 = 4 * 1024 * 1024
    assert L.fibatt_fabric_read(fake, mib4 + 16, 1, fake, None) == fb.E_INVAL
    assert "multiple of 4 MiB" in L.fibatt_last_error().decode()
    assert L.fibatt_fabric_read(fake, 0, 1, fake, None) == fb.E_INVAL
    assert L.fibatt_fabric_read(fake, mib4, 0, fake, None) == fb.E_INVAL
    assert L.fibatt_fabric_read(None, mib4, 1, fake, None) == fb.E_INVAL
    assert L.fibatt_fabric_read(ctypes.c_void_p(0x10004), mib4, 1, fake, None) == fb.E_INVAL
    # fibatt_time_next_call: both or neither event
    assert L.fibatt_time_next_call(fake, None) == fb.E_INVAL
    assert L.fibatt_time_next_call(None, None) == fb.OK
