"""Thin Python binding of libfibatt (include/fibatt.h) via ctypes.

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the current HIP
stream.  If the shared library is missing the first call raises; there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfibatt.so")

OK, E_INVAL, E_RANGE, E_UNSUPPORTED, E_HIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
MAX_HEADS = 128

EXPORTED = ("fibatt_wythoff", "fibatt_wythoff_modified", "fibatt_windows", "fibatt_offsets",
            "fibatt_fwd", "fibatt_bwd", "fibatt_bwd_workspace_floats", "fibatt_fwd_cls",
            "fibatt_bwd_cls", "fibatt_fwd_cls_workspace_floats",
            "fibatt_bwd_cls_workspace_floats", "fibatt_fwd_table", "fibatt_bwd_table",
            "fibatt_fwd_table_workspace_floats", "fibatt_bwd_table_workspace_floats",
            "fibatt_fwd_strided", "fibatt_bwd_strided", "fibatt_bwd_noalloc",
            "fibatt_time_next_call", "fibatt_hbm_stream", "fibatt_fabric_read",
            "fibatt_last_error")


class FibattError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"fibatt error {code}: {message}")
        self.code = code
        self.message = message


class Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("d_h", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("a", ctypes.POINTER(ctypes.c_int32)),
        ("b", ctypes.POINTER(ctypes.c_int32)),
        ("w", ctypes.POINTER(ctypes.c_int32)),
    ]


class TableDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("d_h", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("cls", ctypes.c_int32),
        ("head_ptr", ctypes.POINTER(ctypes.c_int32)),
        ("offs", ctypes.POINTER(ctypes.c_int32)),
        ("offs_device", ctypes.c_void_p),
    ]


class Layout(ctypes.Structure):
    _fields_ = [("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("sn", ctypes.c_int64)]


class Layouts(ctypes.Structure):
    _fields_ = [(n, Layout) for n in ("q", "k", "v", "o", "dout", "dq", "dk", "dv")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m structured_sparse_head_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    L.fibatt_wythoff.argtypes = [ctypes.c_int32, i32p, i32p]
    L.fibatt_wythoff.restype = ctypes.c_int
    L.fibatt_wythoff_modified.argtypes = [ctypes.c_int32, i32p, i32p]
    L.fibatt_wythoff_modified.restype = ctypes.c_int
    L.fibatt_windows.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p]
    L.fibatt_windows.restype = ctypes.c_int
    L.fibatt_offsets.argtypes = [ctypes.c_int32, ctypes.c_int32, i32p, i32p, i32p, i32p, i32p,
                                 ctypes.c_int32]
    L.fibatt_offsets.restype = ctypes.c_int
    L.fibatt_fwd.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp]
    L.fibatt_fwd.restype = ctypes.c_int
    L.fibatt_bwd.argtypes = [ctypes.POINTER(Desc)] + [vp] * 10
    L.fibatt_bwd.restype = ctypes.c_int
    L.fibatt_bwd_workspace_floats.argtypes = [ctypes.POINTER(Desc)]
    L.fibatt_bwd_workspace_floats.restype = ctypes.c_int64
    L.fibatt_fwd_cls.argtypes = [ctypes.POINTER(Desc)] + [vp] * 7
    L.fibatt_fwd_cls.restype = ctypes.c_int
    L.fibatt_bwd_cls.argtypes = [ctypes.POINTER(Desc)] + [vp] * 10
    L.fibatt_bwd_cls.restype = ctypes.c_int
    for name in ("fibatt_fwd_cls_workspace_floats", "fibatt_bwd_cls_workspace_floats"):
        getattr(L, name).argtypes = [ctypes.POINTER(Desc)]
        getattr(L, name).restype = ctypes.c_int64
    L.fibatt_fwd_table.argtypes = [ctypes.POINTER(TableDesc)] + [vp] * 7
    L.fibatt_fwd_table.restype = ctypes.c_int
    L.fibatt_bwd_table.argtypes = [ctypes.POINTER(TableDesc)] + [vp] * 10
    L.fibatt_bwd_table.restype = ctypes.c_int
    for name in ("fibatt_fwd_table_workspace_floats", "fibatt_bwd_table_workspace_floats"):
        getattr(L, name).argtypes = [ctypes.POINTER(TableDesc)]
        getattr(L, name).restype = ctypes.c_int64
    L.fibatt_fwd_strided.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                     ctypes.POINTER(Layouts)] + [vp] * 7
    L.fibatt_fwd_strided.restype = ctypes.c_int
    L.fibatt_bwd_strided.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                     ctypes.POINTER(Layouts)] + [vp] * 10
    L.fibatt_bwd_strided.restype = ctypes.c_int
    L.fibatt_bwd_noalloc.argtypes = [ctypes.POINTER(Desc)] + [vp] * 9
    L.fibatt_bwd_noalloc.restype = ctypes.c_int
    L.fibatt_time_next_call.argtypes = [vp, vp]
    L.fibatt_time_next_call.restype = ctypes.c_int
    L.fibatt_hbm_stream.argtypes = [ctypes.POINTER(vp), ctypes.c_int32, ctypes.POINTER(vp),
                                    ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp]
    L.fibatt_fabric_read.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp]
    L.fibatt_fabric_read.restype = ctypes.c_int
    L.fibatt_hbm_stream.restype = ctypes.c_int
    L.fibatt_last_error.argtypes = []
    L.fibatt_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != OK:
        raise FibattError(rc, lib().fibatt_last_error().decode())


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(arr: np.ndarray):
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def wythoff(i: int) -> Tuple[int, int]:
    """(a_i, b_i) of Wythoff row i >= 1."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fibatt_wythoff(i, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def wythoff_modified(i: int) -> Tuple[int, int]:
    """README Algorithm 2's modified pair for Wythoff row i >= 1."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fibatt_wythoff_modified(i, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def wythoff_rows(H: int, modified: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(a, b) int32 arrays for tensor heads 0..H-1 (Wythoff rows 1..H, or
    their modified pairs)."""
    row = wythoff_modified if modified else wythoff
    pairs = [row(i) for i in range(1, H + 1)]
    return _i32([p[0] for p in pairs]), _i32([p[1] for p in pairs])


def windows(H: int, w_min: int, w_max: int) -> np.ndarray:
    """Per-head windows interpolated between w_min and w_max."""
    w = np.zeros(H, dtype=np.int32)
    _check(lib().fibatt_windows(H, w_min, w_max, _ptr(w)))
    return w


def offsets(N: int, a, b, w) -> Tuple[np.ndarray, np.ndarray]:
    """CSR offset table (head_ptr[H+1], offs) from the host generator."""
    a, b, w = _i32(a), _i32(b), _i32(w)
    H = len(a)
    head_ptr = np.zeros(H + 1, dtype=np.int32)
    rc = lib().fibatt_offsets(H, N, _ptr(a), _ptr(b), _ptr(w), _ptr(head_ptr), None, 0)
    if rc not in (OK, E_RANGE):
        _check(rc)
    offs = np.zeros(max(int(head_ptr[-1]), 1), dtype=np.int32)
    _check(lib().fibatt_offsets(H, N, _ptr(a), _ptr(b), _ptr(w), _ptr(head_ptr), _ptr(offs),
                                len(offs)))
    return head_ptr, offs[:head_ptr[-1]]


_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

# torch's current HIP stream of a device as a raw handle.  The direct query
# (which torch's own generated code uses) costs well under a microsecond;
# building a Stream object costs about 2 us per call, which matters for
# small problems.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(device) -> int:
    device = torch.device(device)
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None
                           else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


class Fibottention:
    """A fixed problem shape (B, H, N, d_h, dtype) and per-head (a, b, w).

    cls=True selects the class-token mask (fibatt_fwd_cls / fibatt_bwd_cls):
    token 0 attends, and is attended by, every token.
    Keeps the marshalled descriptor so repeated calls cost one ctypes call.
    Tensors are [B, H, N, d_h]; contiguous ones go to fibatt_fwd / fibatt_bwd
    (or the class-token pair), any other views with unit inner stride to
    fibatt_fwd_strided / fibatt_bwd_strided with their strides.
    """

    def __init__(self, B: int, H: int, N: int, d_h: int, dtype: torch.dtype,
                 a: Sequence[int], b: Sequence[int], w: Sequence[int], cls: bool = False):
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}")
        self.shape = (B, H, N, d_h)
        self.dtype = dtype
        self.cls = bool(cls)
        self._a, self._b, self._w = _i32(a), _i32(b), _i32(w)
        if not (len(self._a) == len(self._b) == len(self._w) == H):
            raise ValueError("a, b, w must have H entries")
        self.desc = Desc(B, H, N, d_h, _DTYPES[dtype], _ptr(self._a), _ptr(self._b), _ptr(self._w))
        self._dp = ctypes.byref(self.desc)
        self._lib = lib()

    def _args(self, *tensors):
        for t in tensors:
            if t is None:
                continue
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("tensors must be contiguous device tensors")
        return [None if t is None else t.data_ptr() for t in tensors]

    @staticmethod
    def _layout(t) -> Layout:
        if not t.is_cuda or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("strided tensors must be 4-d device views with unit inner stride")
        return Layout(t.stride(0), t.stride(1), t.stride(2))

    @staticmethod
    def _strided(*tensors) -> bool:
        return any(t is not None and not t.is_contiguous() for t in tensors)

    def _floats(self, fn) -> int:
        n = fn(self._dp)
        if n < 0:
            _check(E_INVAL)
        return int(n)

    def workspace_floats(self) -> int:
        """fp32 elements of the backward's workspace."""
        fn = self._lib.fibatt_bwd_cls_workspace_floats if self.cls else \
            self._lib.fibatt_bwd_workspace_floats
        return self._floats(fn)

    def fwd_workspace_floats(self) -> int:
        """fp32 elements of the forward's workspace (class-token mask only)."""
        return self._floats(self._lib.fibatt_fwd_cls_workspace_floats) if self.cls else 0

    def forward(self, q, k, v, o=None, lse=None, workspace=None, stream: Optional[int] = None):
        """(o, lse).  o in the input dtype, lse fp32 [B, H, N]."""
        for t in (q, k, v):
            if tuple(t.shape) != self.shape or t.dtype != self.dtype:
                raise ValueError(f"expected {self.shape} {self.dtype}, got {tuple(t.shape)} {t.dtype}")
        if o is None:
            o = torch.empty(self.shape, dtype=self.dtype, device=q.device)
        if lse is None:
            lse = torch.empty(self.shape[:3], dtype=torch.float32, device=q.device)
        if self._strided(q, k, v, o):
            if tuple(o.shape) != self.shape or o.dtype != self.dtype:
                raise ValueError(f"o must be {self.shape} {self.dtype}")
            ls = Layouts()
            ls.q, ls.k, ls.v, ls.o = (self._layout(t) for t in (q, k, v, o))
            n = self.fwd_workspace_floats()
            if workspace is None and n > 0:
                workspace = torch.empty(n, dtype=torch.float32, device=q.device)
            ptrs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()] + \
                self._args(lse, workspace)
            s = _current_stream(q.device) if stream is None else stream
            _check(self._lib.fibatt_fwd_strided(self._dp, int(self.cls), ctypes.byref(ls), *ptrs,
                                                s))
        elif self.cls:
            n = self.fwd_workspace_floats()
            if workspace is None and n > 0:
                workspace = torch.empty(n, dtype=torch.float32, device=q.device)
            ptrs = self._args(q, k, v, o, lse, workspace)
            s = _current_stream(q.device) if stream is None else stream
            _check(self._lib.fibatt_fwd_cls(self._dp, *ptrs, s))
        else:
            ptrs = self._args(q, k, v, o, lse)
            s = _current_stream(q.device) if stream is None else stream
            _check(self._lib.fibatt_fwd(self._dp, *ptrs, s))
        return o, lse

    def backward(self, q, k, v, lse, do, dq=None, dk=None, dv=None, workspace=None,
                 stream: Optional[int] = None):
        """(dq, dk, dv) in fp32; lse is the forward's."""
        for t in (q, k, v, do):
            if tuple(t.shape) != self.shape or t.dtype != self.dtype:
                raise ValueError(f"expected {self.shape} {self.dtype}, got {tuple(t.shape)} {t.dtype}")
        dev = q.device
        mk = lambda: torch.empty(self.shape, dtype=torch.float32, device=dev)  # noqa: E731
        dq = mk() if dq is None else dq
        dk = mk() if dk is None else dk
        dv = mk() if dv is None else dv
        if workspace is None:
            workspace = torch.empty(self.workspace_floats(), dtype=torch.float32, device=dev)
        if self._strided(q, k, v, do, dq, dk, dv):
            for t in (dq, dk, dv):
                if tuple(t.shape) != self.shape or t.dtype != torch.float32:
                    raise ValueError(f"dq, dk, dv must be {self.shape} float32")
            ls = Layouts()
            ls.q, ls.k, ls.v, ls.dout, ls.dq, ls.dk, ls.dv = (
                self._layout(t) for t in (q, k, v, do, dq, dk, dv))
            ptrs = [t.data_ptr() for t in (q, k, v)] + self._args(lse) + \
                [t.data_ptr() for t in (do, dq, dk, dv)] + self._args(workspace)
            s = _current_stream(dev) if stream is None else stream
            _check(self._lib.fibatt_bwd_strided(self._dp, int(self.cls), ctypes.byref(ls), *ptrs,
                                                s))
            return dq, dk, dv
        ptrs = self._args(q, k, v, lse, do, dq, dk, dv, workspace)
        s = _current_stream(dev) if stream is None else stream
        fn = self._lib.fibatt_bwd_cls if self.cls else self._lib.fibatt_bwd
        _check(fn(self._dp, *ptrs, s))
        return dq, dk, dv

    def backward_noalloc(self, q, k, v, lse, do, dq, dk, dv, stream: Optional[int] = None):
        """fibatt_bwd_noalloc: the backward with the library's fixed scratch
        array instead of a workspace (dense tensors, no class-token mask); the
        caller passes the outputs, and nothing is allocated on the device."""
        if self.cls:
            raise ValueError("fibatt_bwd_noalloc has no class-token variant")
        for t in (q, k, v, do):
            if tuple(t.shape) != self.shape or t.dtype != self.dtype:
                raise ValueError(f"expected {self.shape} {self.dtype}, got {tuple(t.shape)} {t.dtype}")
        for t in (dq, dk, dv):
            if tuple(t.shape) != self.shape or t.dtype != torch.float32:
                raise ValueError(f"dq, dk, dv must be {self.shape} float32")
        ptrs = self._args(q, k, v, lse, do, dq, dk, dv)
        s = _current_stream(q.device) if stream is None else stream
        _check(self._lib.fibatt_bwd_noalloc(self._dp, *ptrs, s))
        return dq, dk, dv


class FibottentionTable:
    """Heads given by an explicit distance table (fibatt_fwd_table /
    fibatt_bwd_table): head h attends the distances offs[head_ptr[h] ..
    head_ptr[h+1]).  The table is copied to the device once, here."""

    def __init__(self, B: int, H: int, N: int, d_h: int, dtype: torch.dtype, head_ptr, offs,
                 cls: bool = False, device=None):
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}")
        self.shape = (B, H, N, d_h)
        self.dtype = dtype
        self._ptr, self._offs = _i32(head_ptr), _i32(offs)
        if len(self._ptr) != H + 1:
            raise ValueError("head_ptr must have H + 1 entries")
        dev = torch.device("cuda:0") if device is None else torch.device(device)
        # one padding entry keeps the device copy non-empty
        self._offs_dev = torch.from_numpy(
            np.concatenate([self._offs, np.zeros(1, dtype=np.int32)])).to(dev)
        assert self._offs_dev.dtype == torch.int32
        self.desc = TableDesc(B, H, N, d_h, _DTYPES[dtype], int(bool(cls)), _ptr(self._ptr),
                              _ptr(self._offs), self._offs_dev.data_ptr())
        self._dp = ctypes.byref(self.desc)
        self._lib = lib()

    _args = Fibottention._args

    def _floats(self, fn) -> int:
        n = fn(self._dp)
        if n < 0:
            _check(E_INVAL)
        return int(n)

    def _shapes(self, *tensors):
        for t in tensors:
            if tuple(t.shape) != self.shape or t.dtype != self.dtype:
                raise ValueError(f"expected {self.shape} {self.dtype}, got {tuple(t.shape)} {t.dtype}")
            if t.device != self._offs_dev.device:
                raise ValueError(f"tensors must be on {self._offs_dev.device}, where the table is")

    def forward(self, q, k, v, o=None, lse=None, workspace=None, stream: Optional[int] = None):
        """(o, lse) as Fibottention.forward."""
        self._shapes(q, k, v)
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(self.shape[:3], dtype=torch.float32, device=q.device)
        n = self._floats(self._lib.fibatt_fwd_table_workspace_floats)
        if workspace is None and n > 0:
            workspace = torch.empty(n, dtype=torch.float32, device=q.device)
        ptrs = self._args(q, k, v, o, lse, workspace)
        s = _current_stream(q.device) if stream is None else stream
        _check(self._lib.fibatt_fwd_table(self._dp, *ptrs, s))
        return o, lse

    def backward(self, q, k, v, lse, do, workspace=None, stream: Optional[int] = None):
        """fp32 (dq, dk, dv) as Fibottention.backward."""
        self._shapes(q, k, v, do)
        dev = q.device
        dq, dk, dv = (torch.empty(self.shape, dtype=torch.float32, device=dev) for _ in range(3))
        if workspace is None:
            n = self._floats(self._lib.fibatt_bwd_table_workspace_floats)
            workspace = torch.empty(n, dtype=torch.float32, device=dev)
        ptrs = self._args(q, k, v, lse, do, dq, dk, dv, workspace)
        s = _current_stream(dev) if stream is None else stream
        _check(self._lib.fibatt_bwd_table(self._dp, *ptrs, s))
        return dq, dk, dv


def forward(q, k, v, a, b, w, cls: bool = False):
    """One-shot forward for q, k, v of shape [B, H, N, d_h] on the GPU."""
    B, H, N, d = q.shape
    return Fibottention(B, H, N, d, q.dtype, a, b, w, cls=cls).forward(q, k, v)


def backward(q, k, v, lse, do, a, b, w, cls: bool = False):
    """One-shot backward; returns fp32 (dq, dk, dv)."""
    B, H, N, d = q.shape
    return Fibottention(B, H, N, d, q.dtype, a, b, w, cls=cls).backward(q, k, v, lse, do)


class FibottentionFunction(torch.autograd.Function):
    """autograd wrapper: y = Fibottention(q, k, v); gradients from fibatt_bwd
    (or fibatt_bwd_cls with cls=True)."""

    @staticmethod
    def forward(ctx, q, k, v, a, b, w, cls=False):
        B, H, N, d = q.shape
        op = Fibottention(B, H, N, d, q.dtype, a, b, w, cls=cls)
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = op.forward(q, k, v)
        ctx.op = op
        ctx.save_for_backward(q, k, v, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, lse = ctx.saved_tensors
        dq, dk, dv = ctx.op.backward(q, k, v, lse, do.to(q.dtype).contiguous())
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None


class FibottentionQKVFunction(torch.autograd.Function):
    """autograd wrapper over a fused projection: qkv [B, N, 3, H, d_h] (Q, K
    and V of every head side by side, as X [W^Q | W^K | W^V] lays them out)
    -> O [B, N, H, d_h], ready for the output projection.  The kernels read
    and write the strided head views directly (fibatt_fwd_strided /
    fibatt_bwd_strided), so no head split or merge copies are made; the
    gradient comes back as one fp32 [B, N, 3, H, d_h] buffer."""

    @staticmethod
    def _heads(t):
        return [t[:, :, i].permute(0, 2, 1, 3) for i in range(3)]

    @staticmethod
    def forward(ctx, qkv, a, b, w, cls=False):
        B, N, three, H, d = qkv.shape
        if three != 3 or not qkv.is_contiguous():
            raise ValueError("qkv must be a contiguous [B, N, 3, H, d_h] tensor")
        op = Fibottention(B, H, N, d, qkv.dtype, a, b, w, cls=cls)
        q, k, v = FibottentionQKVFunction._heads(qkv)
        o = torch.empty(B, N, H, d, dtype=qkv.dtype, device=qkv.device)
        _, lse = op.forward(q, k, v, o=o.permute(0, 2, 1, 3))
        ctx.op = op
        ctx.save_for_backward(qkv, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        qkv, lse = ctx.saved_tensors
        B, N, _, H, d = qkv.shape
        q, k, v = FibottentionQKVFunction._heads(qkv)
        do = do.to(qkv.dtype).contiguous().permute(0, 2, 1, 3)
        g = torch.empty(B, N, 3, H, d, dtype=torch.float32, device=qkv.device)
        dq, dk, dv = FibottentionQKVFunction._heads(g)
        ctx.op.backward(q, k, v, lse, do, dq=dq, dk=dk, dv=dv)
        return g.to(qkv.dtype), None, None, None, None


def time_next_call(start_event: int, stop_event: int) -> None:
    """fibatt_time_next_call: bind two hipEvent_t handles to the kernels of
    the next call on this thread (measurement aid)."""
    _check(lib().fibatt_time_next_call(start_event, stop_event))


def hbm_stream(src: Sequence[torch.Tensor], dst: Sequence[torch.Tensor], nbytes: int,
               dst_scale: int = 1, stream: Optional[int] = None) -> None:
    """fibatt_hbm_stream: read `nbytes` from each tensor of src and write
    dst_scale * nbytes to each of dst (the HBM byte mix of a pass, nothing
    else); measurement aid."""
    for t in list(src) + list(dst):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("hbm_stream takes contiguous device tensors")
    for t in src:
        if t.numel() * t.element_size() < nbytes:
            raise ValueError("a source tensor is smaller than nbytes")
    for t in dst:
        if t.numel() * t.element_size() < dst_scale * nbytes:
            raise ValueError("a destination tensor is smaller than dst_scale * nbytes")
    S = (ctypes.c_void_p * len(src))(*[t.data_ptr() for t in src])
    D = (ctypes.c_void_p * len(dst))(*[t.data_ptr() for t in dst])
    s = _current_stream(src[0].device) if stream is None else stream
    _check(lib().fibatt_hbm_stream(S, len(src), D, len(dst), nbytes, dst_scale, s))


FABRIC_OUT_BYTES = 16 * 8 * 128


def fabric_read(buf: torch.Tensor, passes: int, out: torch.Tensor,
                stream: Optional[int] = None) -> None:
    """fibatt_fabric_read: every XCD reads all of `buf` (contiguous device
    tensor, a multiple of 4 MiB) `passes` times; `out` receives one 16-byte
    xor per workgroup (FABRIC_OUT_BYTES).  Measurement aid."""
    for t in (buf, out):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("fabric_read takes contiguous device tensors")
    if out.numel() * out.element_size() < FABRIC_OUT_BYTES:
        raise ValueError("out is smaller than FABRIC_OUT_BYTES")
    s = _current_stream(buf.device) if stream is None else stream
    _check(lib().fibatt_fabric_read(buf.data_ptr(), buf.numel() * buf.element_size(), passes,
                                    out.data_ptr(), s))
