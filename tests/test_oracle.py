"""Pins for the CPU oracle: closed forms, invariants, brute force and library
routines that the oracle's own code does not use.  CPU only."""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Wythoff rows
# --------------------------------------------------------------------------

def _floor_phi_decimal(n: int) -> int:
    getcontext().prec = 60
    phi = (Decimal(1) + Decimal(5).sqrt()) / 2
    return int((Decimal(n) * phi).to_integral_value(rounding="ROUND_FLOOR"))


def test_wythoff_rows_match_floor_formula_in_decimal():
    # Standard closed form a_i = floor(floor(i phi) phi), b_i = floor(floor(i phi) phi^2),
    # evaluated with 60-digit decimals (no Zeckendorf involved).
    getcontext().prec = 60
    phi = (Decimal(1) + Decimal(5).sqrt()) / 2
    for i in range(1, 301):
        p = _floor_phi_decimal(i)
        a = int((Decimal(p) * phi).to_integral_value(rounding="ROUND_FLOOR"))
        b = int((Decimal(p) * phi * phi).to_integral_value(rounding="ROUND_FLOOR"))
        assert oracle.wythoff_row(i) == (a, b), i


def test_wythoff_row1_is_fibonacci():
    a, b = oracle.wythoff_row(1)
    assert [oracle.fib_term(a, b, n) for n in range(1, 11)] == [1, 2, 3, 5, 8, 13, 21, 34, 55, 89]


def test_fib_term_closed_form_matches_the_recurrence():
    # The closed form a F_{n-2} + b F_{n-1} against the defining recurrence
    # (first term a, second b, then sums of the two before), run here.
    rng = np.random.default_rng(3)
    for _ in range(200):
        a, b = int(rng.integers(0, 10 ** 6)), int(rng.integers(1, 10 ** 6))
        x, y = a, b
        for n in range(1, 60):
            assert oracle.fib_term(a, b, n) == x, (a, b, n)
            x, y = y, x + y


def test_fib_offsets_window_and_duplicates():
    # The window is inclusive and keeps no term above it (the first term that
    # reaches w is kept only when it equals w); repeated terms count once.
    assert oracle.fib_offsets(1, 2, 10, 100) == [1, 2, 3, 5, 8]
    assert oracle.fib_offsets(1, 2, 13, 100) == [1, 2, 3, 5, 8, 13]
    assert oracle.fib_offsets(1, 2, 100, 9) == [1, 2, 3, 5, 8]        # N - 1 = 8
    assert oracle.fib_offsets(0, 1, 20, 100) == [0, 1, 2, 3, 5, 8, 13]  # 1 appears twice
    assert oracle.fib_offsets(3, 3, 20, 100) == [3, 6, 9, 15]          # 3, 3, 6, 9, 15, 24
    assert oracle.fib_offsets(7, 2, 10, 100) == [2, 7, 9]              # first term above the second
    assert oracle.fib_offsets(50, 1, 40, 100) == [1]                   # 50, 1, 51, ...


def test_wythoff_rows_partition_the_positive_integers():
    # Paper, Wythoff array paragraph: rows do not overlap and contain every
    # positive integer exactly once.  Rows 1..R cover every integer below the
    # first term of row R+1.
    R = 199
    limit = oracle.wythoff_row(R + 1)[0] - 1
    seen = {}
    for i in range(1, R + 1):
        a, b = oracle.wythoff_row(i)
        for x in oracle.fib_offsets(a, b, limit, limit + 1):
            assert x not in seen, (x, i, seen.get(x))
            seen[x] = i
    assert sorted(seen) == list(range(1, limit + 1))


def test_wythoff_first_column_is_mex_and_gap_is_floor_i_phi():
    used = set()
    for i in range(1, 120):
        a, b = oracle.wythoff_row(i)
        mex = 1
        while mex in used:
            mex += 1
        assert a == mex
        assert b - a == _floor_phi_decimal(i)
        used.update(oracle.fib_offsets(a, b, 10 ** 6, 10 ** 6 + 1))


# --------------------------------------------------------------------------
# Offsets
# --------------------------------------------------------------------------

def _row_of(d: int, first_col_rank) -> int:
    # Shift d's Zeckendorf representation down until it uses F_2 = 1; the
    # result is the first entry of d's row.
    idx = oracle.zeckendorf(d)
    shift = min(idx)
    root = sum(_fib(t - shift) for t in idx)
    return first_col_rank[root]


def _fib(t):
    a, b = 1, 2
    for _ in range(t):
        a, b = b, a + b
    return a


@pytest.mark.parametrize("N,H,wmode", [(197, 12, "N"), (65, 3, "N"), (4097, 16, "N"),
                                       (1569, 12, "mixed"), (300, 20, "small")])
def test_offsets_brute_force_membership(N, H, wmode):
    # For Wythoff heads: d is an offset of head i iff d lies in row i of the
    # array (row found by Zeckendorf shifting, independent of Algorithm 1).
    a, b = oracle.wythoff_rows(H)
    rng = np.random.default_rng(7)
    if wmode == "N":
        w = [N] * H
    elif wmode == "mixed":
        w = list(rng.integers((N + 3) // 4, N + 1, size=H))
    else:
        w = list(rng.integers(1, 40, size=H))
    first_col_rank = {oracle.wythoff_row(i)[0]: i for i in range(1, 2000)}
    for h in range(H):
        F = set(oracle.fib_offsets(int(a[h]), int(b[h]), int(w[h]), N))
        lim = min(int(w[h]), N - 1)
        expect = {d for d in range(1, lim + 1) if _row_of(d, first_col_rank) == h + 1}
        assert F == expect, (h, sorted(F), sorted(expect))


def test_offsets_log_bound():
    # O(N log w) claim: |F_i| <= floor(log_phi(w_i / a_i)) + 2.
    phi = (1 + 5 ** 0.5) / 2
    for N, H in [(65, 3), (197, 12), (1569, 12), (4097, 16), (65536, 16)]:
        a, b = oracle.wythoff_rows(H)
        for h in range(H):
            F = oracle.fib_offsets(int(a[h]), int(b[h]), N, N)
            assert len(F) <= math.floor(math.log(N / a[h], phi)) + 2


def test_offsets_vit_b_head_counts():
    a, b = oracle.wythoff_rows(12)
    counts = [len(oracle.fib_offsets(int(a[h]), int(b[h]), 197, 197)) for h in range(12)]
    assert counts == [11, 8, 8, 7, 6, 6, 6, 5, 5, 5, 5, 4]
    # head 1 is the ordinary Fibonacci numbers below N
    assert oracle.fib_offsets(1, 2, 197, 197) == [1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144]


def test_offsets_edge_cases():
    assert oracle.fib_offsets(0, 1, 10, 100) == [0, 1, 2, 3, 5, 8]     # 0 once, 1 once
    assert oracle.fib_offsets(3, 3, 20, 100) == [3, 6, 9, 15]          # duplicate start
    assert oracle.fib_offsets(5, 1, 3, 100) == [1]                      # a > w, b <= w
    assert oracle.fib_offsets(4, 7, 7, 100) == [4, 7]                   # window inclusive
    assert oracle.fib_offsets(4, 7, 6, 100) == [4]
    assert oracle.fib_offsets(1, 2, 1, 100) == [1]
    assert oracle.fib_offsets(1, 2, 50, 1) == []                        # N = 1: no partner
    assert oracle.fib_offsets(0, 1, 50, 1) == [0]
    assert oracle.fib_offsets(9, 15, 65, 8) == []                       # all offsets >= N
    with pytest.raises(ValueError):
        oracle.fib_offsets(0, 0, 5, 10)


def test_offset_table_csr():
    a, b = oracle.wythoff_rows(3)
    ptr, offs = oracle.offset_table(65, a, b, [65, 65, 65])
    assert list(ptr) == [0, 9, 15, 20]
    assert list(offs[:9]) == [1, 2, 3, 5, 8, 13, 21, 34, 55]


# --------------------------------------------------------------------------
# Support set
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 5, 17, 65])
def test_support_pair_count_closed_form_and_symmetry(N):
    a, b = oracle.wythoff_rows(6)
    for h in range(6):
        F = oracle.fib_offsets(int(a[h]), int(b[h]), N, N)
        m = oracle.support_mask(N, F)
        assert (m == m.T).all()
        assert m.sum() == sum(2 * (N - f) for f in F)
        assert not m.diagonal().any()
    F0 = oracle.fib_offsets(0, 1, N, N)
    assert oracle.support_mask(N, F0).sum() == N + sum(2 * (N - f) for f in F0 if f > 0)


def test_pages_two_percent_figure():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as fh:
        g = json.load(fh)["kept_interactions"]
    N, H, w_max = 197, 12, g["w_max"]
    a, b = oracle.wythoff_rows(H)
    shares = []
    for w_min in range(1, w_max + 1):
        ws = oracle.window_sizes(H, w_min, w_max)
        pairs = sum(sum(2 * (N - f) for f in oracle.fib_offsets(int(a[h]), int(b[h]), ws[h], N))
                    for h in range(H))
        shares.append(100.0 * pairs / (H * N * N))
    assert any(round(s) == g["value_percent"] for s in shares)
    assert all(s < 5 for s in shares)


def test_wythoff_modified_is_extended_array_columns():
    # The recurrence run two steps back from row i lands on columns -1 and 0
    # of the extended Wythoff array: i - 1 and floor(i phi).  Checked against
    # a decimal evaluation of floor(i phi), not against the oracle's Zeckendorf
    # construction.
    for i in range(1, 1501):
        a_m, b_m = oracle.wythoff_row_modified(i)
        assert a_m == i - 1, i
        assert b_m == _floor_phi_decimal(i), i


def test_wythoff_modified_offsets_extend_the_row():
    N = 1000
    for i in range(1, 13):
        a, b = oracle.wythoff_row(i)
        a_m, b_m = oracle.wythoff_row_modified(i)
        plain = set(oracle.fib_offsets(a, b, N, N))
        mod = set(oracle.fib_offsets(a_m, b_m, N, N))
        assert plain <= mod and mod - plain == {a_m, b_m} - plain, i
    # Head 1: 0, 1, 1, 2, 3, ... -> distance 0 joins the support.
    assert oracle.fib_offsets(*oracle.wythoff_row_modified(1), 20, 21) == [0, 1, 2, 3, 5, 8, 13]


def test_window_sizes_interpolate():
    assert oracle.window_sizes(12, 5, 65)[0] == 5
    assert oracle.window_sizes(12, 5, 65)[-1] == 65
    assert oracle.window_sizes(1, 5, 65) == [65]


def _floor_sum(m: int, n: int) -> int:
    """sum_{k=0}^{n} floor(k m / n) by the reciprocity identity
    sum_{k=0}^{n-1} floor(k m / n) = ((m - 1)(n - 1) + gcd(m, n) - 1) / 2,
    plus the last term k = n, which is m."""
    return ((m - 1) * (n - 1) + math.gcd(m, n) - 1) // 2 + m


@pytest.mark.parametrize("h", [2, 3, 5, 7, 12, 16, 33])
def test_window_sizes_steps_and_sum(h):
    # Independent pins of the linear interpolation between w_min and w_max:
    # consecutive windows differ by floor or ceil of (w_max - w_min)/(h - 1),
    # and the sum of the floors equals a number-theoretic closed form.
    for w_min, w_max in [(1, 1), (5, 65), (49, 197), (1, 4097), (100, 65536), (3, 10), (7, 8)]:
        ws = oracle.window_sizes(h, w_min, w_max)
        d = w_max - w_min
        lo, hi = d // (h - 1), -(-d // (h - 1))
        assert ws[0] == w_min and ws[-1] == w_max and len(ws) == h
        assert all(lo <= y - x <= hi for x, y in zip(ws, ws[1:]))
        if d > 0:
            assert sum(ws) == h * w_min + _floor_sum(d, h - 1)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _tiny_case(N, H=4, B=2, d=8, seed=0, wyt=True):
    q, k, v, do = (_rand((B, H, N, d), seed + t) for t in range(4))
    if wyt:
        a, b = oracle.wythoff_rows(H)
        F = [oracle.fib_offsets(int(a[h]), int(b[h]), N, N) for h in range(H)]
    else:
        F = [[0, 1, 3], [2], [0], []][:H]
    masks = np.stack([oracle.support_mask(N, f) for f in F])
    return q, k, v, do, F, masks


@pytest.mark.parametrize("N", [1, 2, 5, 13, 40])
def test_forward_matches_dense_brute_force(N):
    q, k, v, do, F, masks = _tiny_case(N)
    o, lse = oracle.forward(q, k, v, F)
    o2, lse2, P = oracle.dense_forward(q, k, v, masks)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    fin = np.isfinite(lse2)
    assert (np.isfinite(lse) == fin).all()
    np.testing.assert_allclose(lse[fin], lse2[fin], atol=1e-12, rtol=0)


def test_forward_matches_torch_sdpa_fp64():
    N = 40
    q, k, v, do, F, masks = _tiny_case(N, H=5, d=16, seed=3)
    o, lse = oracle.forward(q, k, v, F)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    tm = torch.from_numpy(masks)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm).numpy()
    nonempty = masks.any(-1)[None].repeat(q.shape[0], 0)
    np.testing.assert_allclose(o[nonempty], ref[nonempty], atol=1e-12, rtol=0)
    # logsumexp of the masked scaled scores, by torch
    s = torch.einsum("bhnd,bhmd->bhnm", tq, tk) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~tm, float("-inf"))
    ref_lse = torch.logsumexp(s, -1).numpy()
    np.testing.assert_allclose(lse[nonempty], ref_lse[nonempty], atol=1e-12, rtol=0)


def test_forward_invariants():
    N = 30
    q, k, v, do, F, masks = _tiny_case(N, H=4, d=8, seed=5)
    o, lse, P = oracle.dense_forward(q, k, v, masks)
    rows = masks.any(-1)
    for bb in range(q.shape[0]):
        for h in range(4):
            pp = P[bb, h]
            assert (pp >= 0).all()
            assert (pp[~masks[h]] == 0).all()
            np.testing.assert_allclose(pp.sum(-1)[rows[h]], 1.0, atol=1e-14)
            for j in range(N):
                keys = np.nonzero(masks[h, j])[0]
                if len(keys):
                    assert (o[bb, h, j] <= v[bb, h, keys].max(0) + 1e-12).all()
                    assert (o[bb, h, j] >= v[bb, h, keys].min(0) - 1e-12).all()


def test_forward_special_rows():
    # N = 5 with offsets {4}: rows 0 and 4 see one key each, rows 1..3 none.
    N, d = 5, 8
    q, k, v = (_rand((1, 1, N, d), s) for s in (11, 12, 13))
    o, lse = oracle.forward(q, k, v, [[4]])
    assert (o[0, 0, 1:4] == 0).all() and np.isneginf(lse[0, 0, 1:4]).all()
    assert np.array_equal(o[0, 0, 0], v[0, 0, 4]) and np.array_equal(o[0, 0, 4], v[0, 0, 0])
    assert lse[0, 0, 0] == pytest.approx(q[0, 0, 0] @ k[0, 0, 4] / math.sqrt(d), abs=1e-14)
    # two keys: P is a sigmoid of the score difference
    N = 3
    q, k, v = (_rand((1, 1, N, d), s) for s in (21, 22, 23))
    o, lse = oracle.forward(q, k, v, [[1]])
    s0 = q[0, 0, 1] @ k[0, 0, 0] / math.sqrt(d)
    s2 = q[0, 0, 1] @ k[0, 0, 2] / math.sqrt(d)
    p0 = 1 / (1 + math.exp(s2 - s0))
    np.testing.assert_allclose(o[0, 0, 1], p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 2], atol=1e-14)


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 5, 13, 40])
def test_backward_matches_dense_brute_force(N):
    q, k, v, do, F, masks = _tiny_case(N, seed=9)
    g = oracle.backward(q, k, v, do, F)
    g2 = oracle.dense_backward(q, k, v, do, masks)
    for x, y in zip(g, g2):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)


def test_backward_matches_torch_autograd_fp64():
    N = 33
    q, k, v, do, F, masks = _tiny_case(N, H=4, d=16, seed=4)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    m = torch.from_numpy(masks)[None]
    s = s.masked_fill(~m, float("-inf"))
    p = torch.softmax(s, -1)
    p = torch.where(m.any(-1, keepdim=True), p, torch.zeros_like(p))
    out = torch.matmul(p, tv)
    out.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.backward(q, k, v, do, F)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


def test_backward_finite_differences():
    N, d = 12, 4
    q, k, v, do, F, masks = _tiny_case(N, H=3, B=1, d=d, seed=17)
    dq, dk, dv = oracle.backward(q, k, v, do, F)
    eps = 1e-6
    rng = np.random.default_rng(0)

    def loss(q_, k_, v_):
        return float((oracle.forward(q_, k_, v_, F)[0] * do).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in q.shape)
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += eps
            up = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * eps
            dn = loss(args["q"], args["k"], args["v"])
            assert (up - dn) / (2 * eps) == pytest.approx(grad[idx], abs=1e-7), (name, idx)


def test_backward_invariants():
    N = 50
    q, k, v, do, F, masks = _tiny_case(N, H=4, d=8, seed=23)
    dq, dk, dv = oracle.backward(q, k, v, do, F)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    nonempty = masks.any(-1)
    for h in range(4):
        np.testing.assert_allclose(dv[:, h].sum(axis=1), do[:, h][:, nonempty[h]].sum(axis=1),
                                   atol=1e-12)
    # rows with no key get no gradient
    q, k, v, do, F, masks = _tiny_case(6, H=4, d=8, seed=2, wyt=False)
    dq, dk, dv = oracle.backward(q, k, v, do, F)
    assert (dq[:, 3] == 0).all() and (dk[:, 3] == 0).all() and (dv[:, 3] == 0).all()


# --------------------------------------------------------------------------
# Class-token variant (README Algorithm 2: row and column 0 of the mask are
# all ones)
# --------------------------------------------------------------------------

def _cls_case(N, B=2, d=8, seed=0):
    """Wythoff heads 1..3 plus a head with the diagonal (a = 0) and one with
    no distance below N (empty Fibonacci support)."""
    q, k, v, do = (_rand((B, 5, N, d), seed + t) for t in range(4))
    a, b = oracle.wythoff_rows(3)
    F = [oracle.fib_offsets(int(a[h]), int(b[h]), N, N) for h in range(3)]
    F.append(oracle.fib_offsets(0, 2, N, N))           # 0, 2, 4, 6, 10, ...
    F.append([f for f in [N + 5] if f <= N - 1])       # nothing in range
    masks = np.stack([oracle.cls_support_mask(N, f) for f in F])
    return q, k, v, do, F, masks


def _torch_masked_attention(q, k, v, masks):
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    m = torch.from_numpy(masks)[None]
    p = torch.softmax(s.masked_fill(~m, float("-inf")), -1)
    return tq, tk, tv, torch.matmul(p, tv), torch.logsumexp(s.masked_fill(~m, float("-inf")), -1)


@pytest.mark.parametrize("N", [1, 2, 5, 13, 40])
def test_cls_forward_matches_dense_brute_force(N):
    q, k, v, do, F, masks = _cls_case(N, seed=N)
    o, lse = oracle.forward(q, k, v, F, cls=True)
    o2, lse2, P = oracle.dense_forward(q, k, v, masks)
    assert np.isfinite(lse).all()           # every row sees at least key 0
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=0)


@pytest.mark.parametrize("N", [1, 2, 5, 13, 40])
def test_cls_backward_matches_dense_brute_force(N):
    q, k, v, do, F, masks = _cls_case(N, seed=100 + N)
    g = oracle.backward(q, k, v, do, F, cls=True)
    g2 = oracle.dense_backward(q, k, v, do, masks)
    for x, y in zip(g, g2):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)


def test_cls_matches_torch_autograd_fp64():
    N = 29
    q, k, v, do, F, masks = _cls_case(N, d=16, seed=41)
    tq, tk, tv, out, lse_t = _torch_masked_attention(q, k, v, masks)
    out.backward(torch.from_numpy(do))
    o, lse = oracle.forward(q, k, v, F, cls=True)
    dq, dk, dv = oracle.backward(q, k, v, do, F, cls=True)
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_t.detach().numpy(), atol=1e-12, rtol=0)
    for x, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(x, t.grad.numpy(), atol=1e-12, rtol=0)


def test_cls_with_every_distance_is_plain_attention():
    # Fib(0, 1) = 0, 1, 1, 2, 3, 5, 8, ...: with N = 4 every distance 0..3 is
    # a term, so both masks are all ones and the result is dense softmax
    # attention (torch's scaled_dot_product_attention without a mask).
    N = 4
    q, k, v, do = (_rand((2, 1, N, 8), 60 + t) for t in range(4))
    F = [oracle.fib_offsets(0, 1, N, N)]
    assert F == [[0, 1, 2, 3]]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v))).numpy()
    for cls in (False, True):
        o, _ = oracle.forward(q, k, v, F, cls=cls)
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    for x, y in zip(oracle.backward(q, k, v, do, F, cls=True), oracle.backward(q, k, v, do, F)):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)


def test_cls_special_rows():
    # Offsets {4} at N = 5: rows 1..3 have no Fibonacci key, so under the
    # class-token mask each sees key 0 only (O = V_0, LSE = its one score).
    N, d = 5, 8
    q, k, v = (_rand((1, 1, N, d), s) for s in (71, 72, 73))
    o, lse = oracle.forward(q, k, v, [[4]], cls=True)
    for j in (1, 2, 3):
        assert np.array_equal(o[0, 0, j], v[0, 0, 0])
        assert lse[0, 0, j] == pytest.approx(q[0, 0, j] @ k[0, 0, 0] / math.sqrt(d), abs=1e-14)
    # row 4 sees key 0 once (4 is an offset), row 0 sees every key
    s = q[0, 0, 0] @ k[0, 0].T / math.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    np.testing.assert_allclose(o[0, 0, 0], p @ v[0, 0], atol=1e-14)
    # one token: the class token attends itself
    o, lse = oracle.forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], [[]], cls=True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])


@pytest.mark.parametrize("N", [1, 2, 7, 60, 197])
def test_cls_pair_count_closed_form(N):
    # |Omega_cls| = |Omega| + 2 (N - 1 - |F n [1, N-1]|) + [0 not in F]
    for F in ([], [0], [1, 2, 3, 5, 8], [0, 2, 4, 6, 10], [4, 7, 11, 18, 29]):
        F = [f for f in F if f <= N - 1]
        base = oracle.support_mask(N, F).sum()
        pos = len([f for f in F if f >= 1])
        want = base + 2 * (N - 1 - pos) + (0 not in F)
        assert oracle.cls_support_mask(N, F).sum() == want


# --------------------------------------------------------------------------
# One attention layer (README Algorithm 3)
# --------------------------------------------------------------------------

def _block_case(B, N, H, dh, seed, F=None):
    c = H * dh
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, c))
    wq, wk, wv, wz = (rng.standard_normal((c, c)) / math.sqrt(c) for _ in range(4))
    dout = rng.standard_normal((B, N, c))
    if F is None:
        a, b = oracle.wythoff_rows(H)
        F = [oracle.fib_offsets(int(a[h]), int(b[h]), N, N) for h in range(H)]
    return x, wq, wk, wv, wz, dout, F


@pytest.mark.parametrize("cls", [False, True])
def test_block_matches_torch_autograd_fp64(cls):
    B, N, H, dh = 2, 23, 3, 8
    x, wq, wk, wv, wz, dout, F = _block_case(B, N, H, dh, seed=7)
    mk = oracle.cls_support_mask if cls else oracle.support_mask
    masks = torch.from_numpy(np.stack([mk(N, f) for f in F]))[None]
    t = {n: torch.from_numpy(a).requires_grad_() for n, a in
         (("x", x), ("wq", wq), ("wk", wk), ("wv", wv), ("wz", wz))}

    def heads(y):
        return y.reshape(B, N, H, dh).permute(0, 2, 1, 3)

    q, k, v = (heads(t["x"] @ t[w]) for w in ("wq", "wk", "wv"))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(dh)
    p = torch.softmax(s.masked_fill(~masks, float("-inf")), -1)
    p = torch.where(masks.any(-1, keepdim=True), p, torch.zeros_like(p))
    z = torch.matmul(p, v).permute(0, 2, 1, 3).reshape(B, N, H * dh)
    out = z @ t["wz"]
    out.backward(torch.from_numpy(dout))
    ref = oracle.block_forward(x, wq, wk, wv, wz, F, cls=cls)
    np.testing.assert_allclose(ref, out.detach().numpy(), atol=1e-12, rtol=0)
    grads = oracle.block_backward(x, wq, wk, wv, wz, dout, F, cls=cls)
    for g, n in zip(grads, ("x", "wq", "wk", "wv", "wz")):
        np.testing.assert_allclose(g, t[n].grad.numpy(), atol=1e-11, rtol=0, err_msg=n)


def test_block_with_every_distance_is_torch_multihead_attention():
    # Fib(0, 1) covers every distance 0..3 at N = 4: the layer is plain
    # multi-head attention, here torch.nn.MultiheadAttention without biases.
    B, N, H, dh = 3, 4, 2, 8
    c = H * dh
    F = [oracle.fib_offsets(0, 1, N, N)] * H
    x, wq, wk, wv, wz, dout, _ = _block_case(B, N, H, dh, seed=8, F=F)
    mha = torch.nn.MultiheadAttention(c, H, bias=False, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T])))
        mha.out_proj.weight.copy_(torch.from_numpy(wz.T))
    tx = torch.from_numpy(x).requires_grad_()
    out, _ = mha(tx, tx, tx, need_weights=False)
    out.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(oracle.block_forward(x, wq, wk, wv, wz, F),
                               out.detach().numpy(), atol=1e-12, rtol=0)
    dx = oracle.block_backward(x, wq, wk, wv, wz, dout, F)[0]
    np.testing.assert_allclose(dx, tx.grad.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("F", [
    [[3, 6, 9, 12], [0, 5, 10, 15, 20]],                 # constant dilation c n
    [[1, 2, 4, 8, 16, 32], [0, 1, 2, 4, 8, 16, 32]],     # exponential 2^n
    [list(range(1, 12)), []],                           # sliding window, empty head
])
def test_dilation_tables_match_dense_brute_force(F):
    N = 37
    q, k, v, do = (_rand((2, len(F), N, 8), 200 + t) for t in range(4))
    masks = np.stack([oracle.support_mask(N, f) for f in F])
    o, lse = oracle.forward(q, k, v, F)
    o2, lse2, _ = oracle.dense_forward(q, k, v, masks)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    for x, y in zip(oracle.backward(q, k, v, do, F), oracle.dense_backward(q, k, v, do, masks)):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)
