"""The measurement aids of the library on the GPU: fibatt_hbm_stream moves
the bytes it says (every written unit is the xor of the units read),
fibatt_fabric_read reads every unit of its buffer once per pass on every XCD
(each workgroup's xor is that of the units it strides over), and
fibatt_time_next_call brackets exactly one call's kernels (its time lies
inside the time of events recorded around the call, and the binding is gone
afterwards)."""

import ctypes

import pytest
import torch

import structured_sparse_head_amd as fa

pytestmark = pytest.mark.gpu


def _rand_words(n, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), generator=g, device="cuda:0",
                         dtype=torch.int32)


@pytest.mark.parametrize("n_src,n_dst,scale", [(3, 1, 1), (4, 3, 2), (1, 1, 1), (2, 4, 2)])
def test_hbm_stream_writes_the_xor_of_its_reads(n_src, n_dst, scale):
    words = 3 * 1024 * 1024 + 4 * 77  # not a multiple of the grid's stride
    src = [_rand_words(words, 7 + i) for i in range(n_src)]
    dst = [torch.zeros(words * scale, dtype=torch.int32, device="cuda:0") for _ in range(n_dst)]
    fa.hbm_stream(src, dst, words * 4, scale)
    torch.cuda.synchronize()
    x = src[0].clone()
    for s in src[1:]:
        x ^= s
    for d in dst:
        assert torch.equal(d[:words], x)
        if scale == 2:
            pat = torch.tensor([1, 2, 3, 4], dtype=torch.int32, device="cuda:0").repeat(words // 4)
            assert torch.equal(d[words:], x ^ pat)


@pytest.mark.parametrize("mib,passes", [(4, 1), (12, 1), (8, 2), (4, 3)])
def test_fabric_read_xors_every_unit(mib, passes):
    words = mib * 1024 * 1024 // 4
    buf = _rand_words(words, 100 + mib)
    out = torch.full((fa.FABRIC_OUT_BYTES // 4,), -1, dtype=torch.int32, device="cuda:0")
    fa.fabric_read(buf, passes, out)
    torch.cuda.synchronize()
    # Workgroup b (XCD b % 8, index k = b // 8 of 128) reads the 2048-unit
    # chunks c with c % 128 == k; its xor over an even number of passes is 0.
    r = buf.view(-1, 128, 2048, 4)
    x = r[0].clone()
    for i in range(1, r.shape[0]):
        x ^= r[i]
    while x.shape[1] > 1:
        h = x.shape[1] // 2
        x = x[:, :h] ^ x[:, h:]
    x = x[:, 0]  # [128, 4]
    if passes % 2 == 0:
        x = torch.zeros_like(x)
    got = out.view(-1, 4)
    assert got.shape[0] == 8 * 128
    for b in range(8 * 128):
        assert torch.equal(got[b], x[b // 8]), b


def _events(n):
    rt = ctypes.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                       ctypes.c_void_p]
    out = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
        out.append(e.value)

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value
    return out, elapsed


def test_time_next_call_brackets_one_call():
    B, H, N, d = 32, 12, 197, 64
    a, b = fa.wythoff_rows(H)
    op = fa.Fibottention(B, H, N, d, torch.bfloat16, a, b, [N] * H)
    q, k, v, do = (torch.randn(B, H, N, d, device="cuda:0").to(torch.bfloat16) for _ in range(4))
    o, lse = op.forward(q, k, v)
    (s, e), elapsed = _events(2)
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    outer0.record()
    fa.time_next_call(s, e)
    op.backward(q, k, v, lse, do)
    outer1.record()
    torch.cuda.synchronize()
    inner = elapsed(s, e)
    assert 0.0 < inner <= outer0.elapsed_time(outer1) + 1e-3
    # the binding was used up: another call leaves the events alone
    op.forward(q, k, v)
    torch.cuda.synchronize()
    assert elapsed(s, e) == inner
