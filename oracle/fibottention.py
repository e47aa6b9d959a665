"""CPU oracle for Fibottention sparse multi-head attention -- TEST INFRASTRUCTURE.

This module is the parity authority for the HIP library in
``structured_sparse_head_amd``.  It is plain, slow and written to be checked
by eye against the method's definition.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.  It shares no code with the HIP path
(no common headers, helpers, tables or generators) and imports nothing from
it.

All floating-point work is fp64 numpy.  Callers hand in the exact values the
GPU sees (for bf16 workloads: the bf16-rounded values, widened to fp64).

Sources (page titles; no other material is used):

* "Fibottention: Inceptive Visual Representation Learning with Diverse
  Attention Across Heads" (arXiv 2406.19391), method section: the sparse
  attention matrix restricted to a support set Omega with the -inf indicator
  (eq. (1) and the Hadamard-product form after it), the dilation sequence and
  window 1 <= w <= N, the generalized Fibonacci support set
  Omega_w^{Fib(a,b)} = {(j,k) : |j-k| in Fib(a,b), |j-k| <= w}, the Wythoff
  array choice of (a_i, b_i), the per-head support Omega_i (eq. (3)) and the
  window interpolation between w_min and w_max.
* The project README of Charlotte-CharMLab/Fibottention: Algorithm 1
  (generalized Fibonacci sequence under a window constraint), Algorithm 2
  (Wythoff rows, the modified pairs) and Algorithm 3 (masked scores -> row
  softmax -> weighted sum of values).
* "Dilated Neighborhood Attention Transformer", background section: scaled
  dot-product attention softmax(Q K^T / sqrt(d)) V, which fixes the
  1/sqrt(d_h) scale.

Readings taken where the pages are garbled or silent:

R1  Row i of the Wythoff array is the standard one: first term
    floor(floor(i*phi)*phi), second term floor(floor(i*phi)*phi^2).  Only this
    reading gives rows that are disjoint and cover every positive integer,
    which is the property the Fibottention paper states for the array.  Here
    the rows are built without phi at all, from Zeckendorf representations
    (see ``wythoff_row``); the tests pin that construction against the floor
    formula evaluated in 60-digit decimal arithmetic.
R2  Head i (1-based) of a layer uses Wythoff row i; tensor head h (0-based)
    uses row h + 1.
R3  Offsets of a head are the distinct terms f of Fib(a, b) with f <= w and
    f <= N - 1: the support set's definition (README Algorithm 1 builds the
    same sequence by repeated sums and stops after the first term that
    reaches w, which can overshoot w by one term; the set definition keeps
    only f <= w).  The oracle takes the terms from their closed form
    f_n = a F_{n-2} + b F_{n-1}.  They are used symmetrically: (j, k) is in
    the support iff |j - k| is an offset.
R4  Off-support scores are -inf (excluded from the softmax); on-support
    scores are Q_j . K_k / sqrt(d_h).  The README's 0/1 multiplicative mask
    and the paper's sign/abs form are read as this.
R5  Softmax runs over keys (each query row is normalised).
R6  A query row with no key in the support gets O = 0, LSE = -inf and
    contributes nothing to any gradient.
R7  An offset of 0 (only possible when a = 0) is the diagonal and counts once.
R8  Token 0 (a CLS token) is an ordinary token: no dense row or column.
    The other reading, README Algorithm 2's mask whose row and column 0 are
    all ones (the class token attends every token and every token attends
    it), is the ``cls=True`` variant of ``forward`` and ``backward``.  There
    the pages index the N patch tokens 1..N behind the class token, so the
    distances between two patches are the same as between their positions
    here; pair (0, 0) is in the support as well.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Wythoff array (paper, method section: "Wythoff array" paragraph, Table 1)
# ---------------------------------------------------------------------------


def _fibonacci_upto(n: int) -> List[int]:
    """Fibonacci numbers 1, 2, 3, 5, 8, ... (F_2, F_3, ...) not exceeding n."""
    fibs = [1, 2]
    while fibs[-1] + fibs[-2] <= n:
        fibs.append(fibs[-1] + fibs[-2])
    return [f for f in fibs if f <= n]


def zeckendorf(n: int) -> List[int]:
    """Zeckendorf representation of n >= 1 as a list of indices into the
    sequence F_2 = 1, F_3 = 2, F_4 = 3, ... (index 0 means F_2).

    Greedy: repeatedly take the largest Fibonacci number that still fits.
    """
    if n < 1:
        raise ValueError("zeckendorf needs n >= 1")
    fibs = _fibonacci_upto(n)
    idx = []
    rest = n
    for t in range(len(fibs) - 1, -1, -1):
        if fibs[t] <= rest:
            idx.append(t)
            rest -= fibs[t]
    assert rest == 0
    return idx


def _from_indices(idx: Sequence[int]) -> int:
    top = max(idx) + 2
    fibs = [1, 2]
    while len(fibs) < top:
        fibs.append(fibs[-1] + fibs[-2])
    return sum(fibs[t] for t in idx)


def fib_successor(n: int) -> int:
    """Shift every Zeckendorf term of n up by one Fibonacci index.

    In the Wythoff array this maps an entry to the entry right of it.
    """
    return _from_indices([t + 1 for t in zeckendorf(n)])


def wythoff_row(i: int) -> Tuple[int, int]:
    """(a_i, b_i): the first two entries of row i >= 1 of the Wythoff array.

    Construction (no golden ratio involved): the first column holds exactly
    the positive integers whose Zeckendorf representation uses F_2 = 1, in
    increasing order; each row continues by the Fibonacci successor.  Row 1
    is therefore 1, 2, 3, 5, 8, ...
    """
    if i < 1:
        raise ValueError("Wythoff rows are numbered from 1")
    a = _first_column(i)[i - 1]
    return a, fib_successor(a)


_FIRST_COLUMN: List[int] = []


def _first_column(count: int) -> List[int]:
    """The first `count` integers whose Zeckendorf representation uses F_2."""
    n = _FIRST_COLUMN[-1] if _FIRST_COLUMN else 0
    while len(_FIRST_COLUMN) < count:
        n += 1
        if min(zeckendorf(n)) == 0:
            _FIRST_COLUMN.append(n)
    return _FIRST_COLUMN


def wythoff_row_modified(i: int) -> Tuple[int, int]:
    """README Algorithm 2, modified branch: from row i's (a, b) take
    b_m = b - a and a_m = a - b_m, i.e. the recurrence run two steps back, so
    Fib(a_m, b_m) = a_m, b_m, a, b, ...  (Head 1 then starts 0, 1.)"""
    a, b = wythoff_row(i)
    b_m = b - a
    return a - b_m, b_m


def wythoff_rows(h: int, modified: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(a, b) int32 arrays for heads 1..h (R2); `modified` selects README
    Algorithm 2's modified pairs."""
    row = wythoff_row_modified if modified else wythoff_row
    pairs = [row(i) for i in range(1, h + 1)]
    a = np.array([p[0] for p in pairs], dtype=np.int32)
    b = np.array([p[1] for p in pairs], dtype=np.int32)
    return a, b


# ---------------------------------------------------------------------------
# Offsets (paper's definition of Omega_w^{Fib(a,b)}; the sequence of README
# Algorithm 1)
# ---------------------------------------------------------------------------


def _fibonacci(n: int) -> int:
    """Standard Fibonacci number F_n for n >= -1 (F_-1 = 1, F_0 = 0, F_1 = 1)."""
    if n == -1:
        return 1
    x, y = 0, 1
    for _ in range(n):
        x, y = y, x + y
    return x


def fib_term(a: int, b: int, n: int) -> int:
    """Term n >= 1 of the generalized Fibonacci sequence Fib(a, b) (first term
    a, second term b, each later term the sum of the two before it), in
    closed form: f_n = a F_{n-2} + b F_{n-1}."""
    if n < 1:
        raise ValueError("terms are numbered from 1")
    return a * _fibonacci(n - 2) + b * _fibonacci(n - 1)


def fib_offsets(a: int, b: int, w: int, n_tokens: int) -> List[int]:
    """Distinct non-negative distances of one head, ascending (R3, R7): the
    members of Fib(a, b) that are at most w (the support set's window) and at
    most N - 1 (no pair is further apart).

    With a >= 0 and b >= 1 the terms from the second on never decrease
    (f_{n+1} = f_n + f_{n-1} >= f_n) and grow without bound, so the members
    up to the limit are f_1 (if small enough) and f_2, f_3, ... up to the
    first term beyond the limit."""
    if a < 0 or b < 1:
        raise ValueError("need a >= 0 and b >= 1 (a = b = 0 gives no sequence)")
    if n_tokens < 1 or w < 1:
        raise ValueError("need N >= 1 and w >= 1")
    limit = min(w, n_tokens - 1)
    members = set()
    n = 1
    while True:
        f = fib_term(a, b, n)
        if n >= 2 and f > limit:
            break
        if f <= limit:
            members.add(f)
        n += 1
    return sorted(members)


def offset_table(n_tokens: int, a: Sequence[int], b: Sequence[int],
                 w: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """CSR table over heads: head_ptr[H+1] and the concatenated offsets."""
    lists = [fib_offsets(int(a[h]), int(b[h]), int(w[h]), n_tokens)
             for h in range(len(a))]
    head_ptr = np.zeros(len(lists) + 1, dtype=np.int32)
    for h, lst in enumerate(lists):
        head_ptr[h + 1] = head_ptr[h] + len(lst)
    offs = np.array([f for lst in lists for f in lst], dtype=np.int32)
    return head_ptr, offs


def window_sizes(h: int, w_min: int, w_max: int) -> List[int]:
    """Paper, method section: w_i = w_min + floor((w_max - w_min)(i - 1)/(h - 1)).

    The formula is undefined for a single head; then w_1 = w_max.
    """
    if h == 1:
        return [w_max]
    return [w_min + ((w_max - w_min) * (i - 1)) // (h - 1) for i in range(1, h + 1)]


def support_mask(n_tokens: int, offsets: Sequence[int]) -> np.ndarray:
    """Dense boolean N x N indicator of Omega = {(j,k): |j-k| in offsets}."""
    allowed = set(int(f) for f in offsets)
    m = np.zeros((n_tokens, n_tokens), dtype=bool)
    for j in range(n_tokens):
        for k in range(n_tokens):
            if abs(j - k) in allowed:
                m[j, k] = True
    return m


def cls_support_mask(n_tokens: int, offsets: Sequence[int]) -> np.ndarray:
    """README Algorithm 2's class-token mask: Omega among tokens 1..N-1 and
    ones in row 0 and column 0."""
    m = support_mask(n_tokens, offsets)
    m[0, :] = True
    m[:, 0] = True
    return m


def _cls_extra_rows(n_tokens: int, offsets: Sequence[int]) -> np.ndarray:
    """Rows j >= 1 that gain key 0 under the class-token mask: those whose
    distance j to token 0 is not one of the head's offsets."""
    dist = set(int(f) for f in offsets)
    return np.array([j >= 1 and j not in dist for j in range(n_tokens)], dtype=bool)


def signed_offsets(offsets: Sequence[int]) -> List[int]:
    """Key displacement k - j for every distance (0 once, f > 0 as -f and +f)."""
    out = []
    for f in offsets:
        if f == 0:
            out.append(0)
        else:
            out.extend((-int(f), int(f)))
    return sorted(out)


# ---------------------------------------------------------------------------
# Forward (paper eq. (1) and (3) with README Algorithm 3's softmax and P.V)
# ---------------------------------------------------------------------------


def _head_scores(q, k, deltas):
    """S[i, b, j] = Q_j . K_{j+delta_i} / sqrt(d) where j + delta_i is a token,
    -inf elsewhere.  q, k: [B, N, d] fp64."""
    B, N, d = q.shape
    S = np.full((len(deltas), B, N), -np.inf)
    scale = 1.0 / math.sqrt(d)
    for i, dl in enumerate(deltas):
        lo, hi = max(0, -dl), min(N, N - dl)
        if lo >= hi:
            continue
        S[i, :, lo:hi] = (q[:, lo:hi, :] * k[:, lo + dl:hi + dl, :]).sum(-1) * scale
    return S


def _head_probs(S):
    """Two-pass row softmax over the offset axis; empty rows give P = 0 (R6)."""
    m = S.max(axis=0, initial=-np.inf)      # [B, N]; no offsets -> -inf
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[None])            # exp(-inf) = 0 off the support
    l = E.sum(axis=0)
    l_safe = np.where(empty, 1.0, l)
    P = E / l_safe[None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return P, lse


def _cls_scores(q, k, extra):
    """One extra score slot per row: Q_j . K_0 / sqrt(d) for the rows that
    gain key 0 under the class-token mask, -inf elsewhere.  Shape [1, B, N]."""
    B, N, d = q.shape
    c = np.full((1, B, N), -np.inf)
    c[0][:, extra] = (q[:, extra, :] * k[:, 0:1, :]).sum(-1) / math.sqrt(d)
    return c


def _dense_row0(q, k):
    """Class-token row: scores of token 0 against every key and their
    softmax.  Returns (P0 [B, N], lse0 [B])."""
    s0 = (q[:, 0:1, :] * k).sum(-1) / math.sqrt(q.shape[-1])   # [B, N]
    m = s0.max(axis=1)
    e = np.exp(s0 - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m + np.log(l)


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
            offsets_per_head: Sequence[Sequence[int]], cls: bool = False):
    """O and LSE (natural log) for q, k, v of shape [B, H, N, d] (fp64).

    Implementation: one pass per signed offset over contiguous slices, then a
    two-pass (max, then exp-sum) softmax.  Returns (o [B,H,N,d], lse [B,H,N]).

    cls=True applies README Algorithm 2's class-token mask: each row j >= 1
    whose distance to token 0 is not an offset gets key 0 as one more score
    slot, and row 0 is a dense softmax over all N keys.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    lse = np.empty((B, H, N))
    for h in range(H):
        deltas = signed_offsets(offsets_per_head[h])
        S = _head_scores(q[:, h], k[:, h], deltas)
        if cls:
            extra = _cls_extra_rows(N, offsets_per_head[h])
            S = np.concatenate([S, _cls_scores(q[:, h], k[:, h], extra)])
            S[:, :, 0] = -np.inf        # row 0 is replaced by the dense row below
        P, lse[:, h] = _head_probs(S)
        for i, dl in enumerate(deltas):
            lo, hi = max(0, -dl), min(N, N - dl)
            if lo < hi:
                o[:, h, lo:hi, :] += P[i, :, lo:hi, None] * v[:, h, lo + dl:hi + dl, :]
        if cls:
            o[:, h] += P[-1][:, :, None] * v[:, h, 0:1, :]
            P0, lse[:, h, 0] = _dense_row0(q[:, h], k[:, h])
            o[:, h, 0] = (P0[:, :, None] * v[:, h]).sum(axis=1)
    return o, lse


# ---------------------------------------------------------------------------
# Backward (exact gradient of the forward; the pages do not spell it out)
# ---------------------------------------------------------------------------


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
             offsets_per_head: Sequence[Sequence[int]], cls: bool = False):
    """dQ, dK, dV of sum(O * dO) for the forward above (fp64).

    With P the support-restricted softmax and dP_jk = dO_j . V_k:
      D_j   = sum_k P_jk dP_jk
      dS_jk = P_jk (dP_jk - D_j)
      dQ_j  = sum_k dS_jk K_k / sqrt(d)
      dK_k  = sum_j dS_jk Q_j / sqrt(d)
      dV_k  = sum_j P_jk dO_j
    The key-side sums are accumulated query-centrically (a slice add per
    signed offset), not key-centrically like the HIP kernels.  cls=True is
    the class-token mask of ``forward``: the extra key-0 slot of rows j >= 1
    and the dense row 0 enter the same formulas.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        deltas = signed_offsets(offsets_per_head[h])
        S = _head_scores(q[:, h], k[:, h], deltas)
        if cls:
            extra = _cls_extra_rows(N, offsets_per_head[h])
            S = np.concatenate([S, _cls_scores(q[:, h], k[:, h], extra)])
            S[:, :, 0] = -np.inf
        P, _ = _head_probs(S)
        dP = np.zeros_like(P)
        for i, dl in enumerate(deltas):
            lo, hi = max(0, -dl), min(N, N - dl)
            if lo < hi:
                dP[i, :, lo:hi] = (do[:, h, lo:hi, :] * v[:, h, lo + dl:hi + dl, :]).sum(-1)
        if cls:
            dP[-1] = (do[:, h] * v[:, h, 0:1, :]).sum(-1)
        D = (P * dP).sum(axis=0)
        dS = P * (dP - D[None])
        for i, dl in enumerate(deltas):
            lo, hi = max(0, -dl), min(N, N - dl)
            if lo >= hi:
                continue
            ks = slice(lo + dl, hi + dl)
            dq[:, h, lo:hi, :] += dS[i, :, lo:hi, None] * k[:, h, ks, :] * scale
            dk[:, h, ks, :] += dS[i, :, lo:hi, None] * q[:, h, lo:hi, :] * scale
            dv[:, h, ks, :] += P[i, :, lo:hi, None] * do[:, h, lo:hi, :]
        if cls:
            # extra key-0 slot of rows j >= 1
            dq[:, h] += dS[-1][:, :, None] * k[:, h, 0:1, :] * scale
            dk[:, h, 0] += (dS[-1][:, :, None] * q[:, h]).sum(axis=1) * scale
            dv[:, h, 0] += (P[-1][:, :, None] * do[:, h]).sum(axis=1)
            # dense row 0
            P0, _ = _dense_row0(q[:, h], k[:, h])                    # [B, N]
            dP0 = (do[:, h, 0:1, :] * v[:, h]).sum(-1)               # [B, N]
            D0 = (P0 * dP0).sum(axis=1)
            dS0 = P0 * (dP0 - D0[:, None])
            dq[:, h, 0] += (dS0[:, :, None] * k[:, h]).sum(axis=1) * scale
            dk[:, h] += dS0[:, :, None] * q[:, h, 0:1, :] * scale
            dv[:, h] += P0[:, :, None] * do[:, h, 0:1, :]
    return dq, dk, dv


# ---------------------------------------------------------------------------
# One attention layer (README Algorithm 3): projections around the core
# ---------------------------------------------------------------------------


def _split_heads(t, h):
    """[B, N, h*d] -> [B, h, N, d] (head i owns columns i*d .. (i+1)*d)."""
    B, N, c = t.shape
    return t.reshape(B, N, h, c // h).transpose(0, 2, 1, 3)


def _merge_heads(t):
    """[B, h, N, d] -> [B, N, h*d]: README Algorithm 3's concatenation Z."""
    B, h, N, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, h * d)


def block_forward(x, wq, wk, wv, wz, offsets_per_head, cls=False):
    """README Algorithm 3 over a batch.  x: [B, N, c]; wq, wk, wv: [c, h*d]
    (head i's W_i^Q, W_i^K, W_i^V are columns i*d .. (i+1)*d); wz: [h*d, c].
    Q_i = X W_i^Q, K_i = X W_i^K, V_i = X W_i^V; Z_i = the head's sparse
    attention (``forward``, with its 1/sqrt(d) scale); O = concat(Z_i) W^Z."""
    x, wq, wk, wv, wz = (np.asarray(t, dtype=np.float64) for t in (x, wq, wk, wv, wz))
    h = len(offsets_per_head)
    q, k, v = (_split_heads(x @ w, h) for w in (wq, wk, wv))
    z, _ = forward(q, k, v, offsets_per_head, cls=cls)
    return _merge_heads(z) @ wz


def block_backward(x, wq, wk, wv, wz, dout, offsets_per_head, cls=False):
    """Gradients of sum(O * dout) for ``block_forward`` with respect to x,
    wq, wk, wv and wz (chain rule through the four projections)."""
    x, wq, wk, wv, wz, dout = (np.asarray(t, dtype=np.float64)
                               for t in (x, wq, wk, wv, wz, dout))
    h = len(offsets_per_head)
    q, k, v = (_split_heads(x @ w, h) for w in (wq, wk, wv))
    z, _ = forward(q, k, v, offsets_per_head, cls=cls)
    zc = _merge_heads(z)
    dwz = np.einsum("bni,bnj->ij", zc, dout)
    dz = _split_heads(dout @ wz.T, h)
    dq, dk, dv = backward(q, k, v, dz, offsets_per_head, cls=cls)
    dQ, dK, dV = (_merge_heads(t) for t in (dq, dk, dv))
    dx = dQ @ wq.T + dK @ wk.T + dV @ wv.T
    dwq, dwk, dwv = (np.einsum("bni,bnj->ij", x, t) for t in (dQ, dK, dV))
    return dx, dwq, dwk, dwv, dwz


# ---------------------------------------------------------------------------
# Dense brute force (tiny N only): the definition with an explicit N x N mask
# ---------------------------------------------------------------------------


def dense_forward(q, k, v, masks):
    """Brute force: full score matrix, -inf off the mask, row softmax, P V.

    masks: [H, N, N] boolean.  Returns (o, lse, P) with P: [B, H, N, N].
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    lse = np.full((B, H, N), -np.inf)
    P = np.zeros((B, H, N, N))
    for bb in range(B):
        for h in range(H):
            S = q[bb, h] @ k[bb, h].T / math.sqrt(d)
            for j in range(N):
                keys = np.nonzero(masks[h, j])[0]
                if len(keys) == 0:
                    continue
                row = S[j, keys]
                mx = row.max()
                e = np.exp(row - mx)
                P[bb, h, j, keys] = e / e.sum()
                lse[bb, h, j] = mx + math.log(e.sum())
            o[bb, h] = P[bb, h] @ v[bb, h]
    return o, lse, P


def dense_backward(q, k, v, do, masks):
    """Brute-force gradients from the dense P (tiny N only)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    _, _, P = dense_forward(q, k, v, masks)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bb in range(B):
        for h in range(H):
            p = P[bb, h]
            dp = do[bb, h] @ v[bb, h].T
            D = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[bb, h] = ds @ k[bb, h] / math.sqrt(d)
            dk[bb, h] = ds.T @ q[bb, h] / math.sqrt(d)
            dv[bb, h] = p.T @ do[bb, h]
    return dq, dk, dv
