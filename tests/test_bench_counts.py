"""The benchmark's counts: Q.K pairs per pass, algorithmic bytes per pass and
algorithmic flops, for the five seeded workloads.

Every fraction the benchmark reports divides by these numbers, so they are
checked here against values worked out by hand beforehand (not recomputed
with the benchmark's own formulas):

* pairs: a head with distance set F attends, in a sequence of N tokens,
  2 (N - f) ordered pairs at each distance f > 0 and N at f = 0 (Fibottention
  paper, method section: the support Omega of a head is symmetric in |j - k|);
* bytes: the forward reads Q, K, V and writes O in the input dtype plus an
  fp32 log-sum-exp per row; the backward reads Q, K, V, dO, O and the
  log-sum-exp and writes fp32 dQ, dK, dV;
* flops: 4 d_h per pair forward (Q.K and P V), 10 d_h backward (the two
  recomputed dots, dS K, P dO and dS Q).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402
from oracle import fibottention as F  # noqa: E402

# workload: (pairs per pass over the batch, forward MB, backward MB,
#            forward flops, backward flops), bytes in units of 1e6
EXPECTED = {
    1: (3_768, 0.40, 0.80, 0.96e6, 2.4e6),
    2: (1_330_944, 78.07, 213.63, 0.341e9, 0.852e9),
    3: (5_024_800, 155.44, 425.36, None, None),
    4: (5_242_840, 135.30, 370.24, 1.342e9, 3.355e9),
    5: (33_037_386, 1077.9, 2957.0, 16.9e9, 42.3e9),
}


def _pairs(wl):
    a, b = F.wythoff_rows(wl.H)
    w = workloads.windows(wl)
    dists = [F.fib_offsets(int(a[h]), int(b[h]), int(w[h]), wl.N) for h in range(wl.H)]
    return wl.B * sum(bench._pairs_per_slab(wl.N, dists))


@pytest.mark.parametrize("num", sorted(EXPECTED))
def test_pairs_bytes_and_flops(num):
    wl = workloads.WORKLOADS[num]
    pairs, fwd_mb, bwd_mb, fwd_fl, bwd_fl = EXPECTED[num]
    got = _pairs(wl)
    assert got == pairs
    es = 2 if wl.dtype == "bf16" else 4
    fwd, bwd, moved = bench.pass_bytes(wl, es)
    digits = 2 if fwd_mb < 1000 else 1
    assert round(fwd / 1e6, digits) == fwd_mb
    assert round(bwd / 1e6, digits) == bwd_mb
    # The backward as built does not read O: one input-dtype row per row less.
    assert bwd - moved == wl.B * wl.H * wl.N * wl.d * es
    for pname, want in (("fwd", fwd_fl), ("bwd", bwd_fl)):
        if want is None:
            continue
        flops = bench.FLOPS_PER_PAIR_ELEM[pname] * wl.d * got
        assert abs(flops - want) <= 0.005 * want, (pname, flops, want)
