"""fibatt_bwd_noalloc (the backward that allocates nothing, scratch in a fixed
device array) against fibatt_bwd with a caller workspace, called through the
C ABI: two calls in a row on the same GPU, the second with a smaller input,
plus the size limit.  Results must be bit for bit those of fibatt_bwd (the
same kernels on the same inputs), and within the backward's tolerance of the
oracle on the small case."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
import structured_sparse_head_amd as fa
from structured_sparse_head_amd import fibatt as fb

pytestmark = pytest.mark.gpu


def _case(B, H, N, d, dtype, seed):
    dev = torch.device("cuda:0")
    a, b = fa.wythoff_rows(H)
    w = np.full(H, N, dtype=np.int32)
    inp = workloads.random_case(seed, B, H, N, d, dtype)
    t = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
    op = fa.Fibottention(B, H, N, d, dtype, a, b, w)
    o, lse = op.forward(t["q"], t["k"], t["v"])
    return op, t, lse, inp, (a, b, w)


def _both(op, t, lse):
    ref = op.backward(t["q"], t["k"], t["v"], lse, t["do"])
    shape = op.shape
    out = [torch.full(shape, float("nan"), dtype=torch.float32, device="cuda:0") for _ in range(3)]
    # straight through the C ABI (the binding method is the same call)
    L = fa.lib()
    ptrs = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), lse.data_ptr(),
            t["do"].data_ptr()] + [x.data_ptr() for x in out]
    rc = L.fibatt_bwd_noalloc(op._dp, *ptrs, torch.cuda.current_stream().cuda_stream)
    assert rc == fa.OK, L.fibatt_last_error()
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
def test_noalloc_matches_workspace_backward_twice(dtype, tol):
    # First call: tile / general kernels that keep D in the scratch array
    # (N = 700); second call, smaller (N = 300, fewer heads).
    for (B, H, N, d, seed) in ((3, 12, 700, 64, 41), (2, 5, 300, 64, 42)):
        op, t, lse, inp, (a, b, w) = _case(B, H, N, d, dtype, seed)
        ref, out = _both(op, t, lse)
        for r, x in zip(ref, out):
            assert torch.equal(r, x), (B, H, N, dtype)
    # the smaller case against the oracle
    F = [oracle.fib_offsets(int(a[h]), int(b[h]), int(w[h]), N) for h in range(H)]
    x64 = {n: inp[n].double().numpy() for n in ("q", "k", "v", "do")}
    rdq, rdk, rdv = oracle.backward(x64["q"], x64["k"], x64["v"], x64["do"], F)
    for got, want in zip(out, (rdq, rdk, rdv)):
        err = np.abs(got.double().cpu().numpy() - want).max()
        assert err <= tol, err


def test_noalloc_vit_shape_and_size_limit():
    op, t, lse, _, _ = _case(4, 12, 197, 64, torch.bfloat16, 43)
    ref, out = _both(op, t, lse)
    for r, x in zip(ref, out):
        assert torch.equal(r, x)
    # B*H*N above FIBATT_NOALLOC_MAX_ROWS is rejected before any work
    arrs = (fb._i32([1]), fb._i32([2]), fb._i32([65]))  # kept alive for the call
    big = fb.Desc(1 << 16, 1, 65, 64, fa.BF16, *[fb._ptr(x) for x in arrs])
    g = t["q"].data_ptr()
    rc = fa.lib().fibatt_bwd_noalloc(ctypes.byref(big), g, g, g, g, g, g, g, g, None)
    assert rc == fa.E_RANGE
    assert b"FIBATT_NOALLOC_MAX_ROWS" in fa.lib().fibatt_last_error()
