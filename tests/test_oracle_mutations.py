"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins
catch every one of them.  Nothing here touches the HIP library."""

import math

import numpy as np
import pytest

import oracle
from oracle import fibottention as fo
import tests.test_oracle as pins


def _expect_pin_failure(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_dropped_scale_is_caught(monkeypatch):
    orig = fo._head_scores

    def unscaled(q, k, deltas):
        return orig(q, k, deltas) * math.sqrt(q.shape[-1])

    monkeypatch.setattr(fo, "_head_scores", unscaled)
    _expect_pin_failure(pins.test_forward_matches_torch_sdpa_fp64)


def test_transposed_operands_are_caught(monkeypatch):
    orig = fo._head_scores
    monkeypatch.setattr(fo, "_head_scores", lambda q, k, deltas: orig(k, q, deltas))
    _expect_pin_failure(pins.test_forward_matches_torch_sdpa_fp64)


def test_one_sided_offsets_are_caught(monkeypatch):
    monkeypatch.setattr(fo, "signed_offsets", lambda offs: sorted(int(f) for f in offs))
    _expect_pin_failure(pins.test_forward_matches_dense_brute_force, 13)


def test_one_sided_mask_is_caught(monkeypatch):
    def upper_only(n, offsets):
        allowed = set(int(f) for f in offsets)
        m = np.zeros((n, n), dtype=bool)
        for j in range(n):
            for k in range(n):
                if k - j in allowed:
                    m[j, k] = True
        return m

    monkeypatch.setattr(oracle, "support_mask", upper_only)
    _expect_pin_failure(pins.test_support_pair_count_closed_form_and_symmetry, 17)


def test_missing_D_term_is_caught(monkeypatch):
    orig_probs = fo._head_probs
    # Returning P unchanged but with the backward's D forced to zero is the
    # classic mistake dS = P * dP; emulate it by zeroing D through P's sum.
    src = fo.backward

    def bad_backward(q, k, v, do, offs):
        dq, dk, dv = src(q, k, v, do, offs)
        # add back P * D K-terms: equivalent to dropping "- D_j"
        q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        o, _ = fo.forward(q64, k64, v64, offs)
        D = (o * do64).sum(-1)
        B, H, N, d = q64.shape
        for h in range(H):
            for dl in fo.signed_offsets(offs[h]):
                lo, hi = max(0, -dl), min(N, N - dl)
                if lo >= hi:
                    continue
                S = fo._head_scores(q64[:, h], k64[:, h], fo.signed_offsets(offs[h]))
                P, _ = orig_probs(S)
                i = fo.signed_offsets(offs[h]).index(dl)
                dq[:, h, lo:hi] += (P[i, :, lo:hi] * D[:, h, lo:hi])[..., None] * \
                    k64[:, h, lo + dl:hi + dl] / math.sqrt(d)
        return dq, dk, dv

    monkeypatch.setattr(oracle, "backward", bad_backward)
    _expect_pin_failure(pins.test_backward_matches_torch_autograd_fp64)


def test_literal_paper_wythoff_formula_is_caught(monkeypatch):
    # The garbled printed form a_i = floor(i phi), b_i = floor(floor(i phi) phi^2)
    phi = (1 + 5 ** 0.5) / 2

    def literal(i):
        a = math.floor(i * phi)
        return a, math.floor(a * phi * phi)

    monkeypatch.setattr(oracle, "wythoff_row", literal)
    _expect_pin_failure(pins.test_wythoff_rows_partition_the_positive_integers)


def test_literal_readme_wythoff_formula_is_caught(monkeypatch):
    phi = (1 + 5 ** 0.5) / 2
    monkeypatch.setattr(oracle, "wythoff_row",
                        lambda i: (int(i * phi * phi), int(i * phi * phi ** 2)))
    _expect_pin_failure(pins.test_wythoff_rows_partition_the_positive_integers)


def test_window_overshoot_is_caught(monkeypatch):
    # Algorithm 1's raw output keeps the first term >= w; forgetting the
    # set definition's |j-k| <= w filter must be caught.
    def overshoot(a, b, w, n):
        terms, k = [], 1
        while not terms or terms[-1] < w or k <= 2:
            terms.append(fo.fib_term(a, b, k))
            k += 1
        return sorted({f for f in terms if f <= n - 1})

    monkeypatch.setattr(oracle, "fib_offsets", overshoot)
    _expect_pin_failure(pins.test_offsets_brute_force_membership, 300, 20, "small")


def test_cls_missing_column_is_caught(monkeypatch):
    # class-token mask without its column: rows j >= 1 never gain key 0
    monkeypatch.setattr(fo, "_cls_extra_rows", lambda n, offs: np.zeros(n, dtype=bool))
    _expect_pin_failure(pins.test_cls_forward_matches_dense_brute_force, 13)


def test_cls_key0_counted_twice_is_caught(monkeypatch):
    # every row j >= 1 gains key 0, also when j is already an offset
    monkeypatch.setattr(fo, "_cls_extra_rows", lambda n, offs: np.arange(n) >= 1)
    _expect_pin_failure(pins.test_cls_forward_matches_dense_brute_force, 13)


def test_cls_row0_counted_twice_is_caught(monkeypatch):
    # the dense class-token row added on top of row 0's own Fibonacci keys in
    # the backward (row 0's offset scores not masked out first)
    src = fo.backward

    def bad_backward(q, k, v, do, offs, cls=False):
        dq, dk, dv = src(q, k, v, do, offs, cls=cls)
        if cls:
            row0 = np.zeros(np.shape(q))
            row0[:, :, 0] = 1.0
            g0 = src(q, k, v, np.asarray(do) * row0, offs, cls=False)
            dq, dk, dv = dq + g0[0], dk + g0[1], dv + g0[2]
        return dq, dk, dv

    monkeypatch.setattr(oracle, "backward", bad_backward)
    _expect_pin_failure(pins.test_cls_backward_matches_dense_brute_force, 13)


def test_block_head_split_interleaved_is_caught(monkeypatch):
    # heads taken as interleaved columns (column c -> head c mod h) instead of
    # contiguous blocks of d columns
    def interleaved(t, h):
        B, N, c = t.shape
        return t.reshape(B, N, c // h, h).transpose(0, 3, 1, 2)

    def merge(t):
        B, h, N, d = t.shape
        return t.transpose(0, 2, 3, 1).reshape(B, N, h * d)

    monkeypatch.setattr(fo, "_split_heads", interleaved)
    monkeypatch.setattr(fo, "_merge_heads", merge)
    _expect_pin_failure(pins.test_block_matches_torch_autograd_fp64, False)


def test_block_missing_value_projection_gradient_is_caught(monkeypatch):
    src = fo.block_backward

    def bad(*args, **kw):
        dx, dwq, dwk, dwv, dwz = src(*args, **kw)
        return dx, dwq, dwk, np.zeros_like(dwv), dwz

    monkeypatch.setattr(oracle, "block_backward", bad)
    _expect_pin_failure(pins.test_block_matches_torch_autograd_fp64, False)


def test_window_round_instead_of_floor_is_caught(monkeypatch):
    # interpolation that rounds to nearest instead of flooring
    def rounded(h, w_min, w_max):
        if h == 1:
            return [w_max]
        return [w_min + int(round((w_max - w_min) * (i - 1) / (h - 1))) for i in range(1, h + 1)]

    monkeypatch.setattr(oracle, "window_sizes", rounded)
    _expect_pin_failure(pins.test_window_sizes_steps_and_sum, 7)
