"""The host layer of the library (csrc/host.cpp: validation, Wythoff rows,
windows, offset table, workspace sizes) built with the host C++ compiler
under AddressSanitizer and UndefinedBehaviorSanitizer, driven through every
error path and checked bit for bit against the oracle.  CPU only.

Pins: the oracle's Wythoff rows, modified pairs, windows and offset table
(themselves pinned in test_oracle.py), and the status codes include/fibatt.h
documents for each invalid argument."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = shutil.which("g++") or shutil.which("clang++")
OK, E_INVAL, E_RANGE, E_UNSUPPORTED = 0, 1, 2, 3

pytestmark = pytest.mark.skipif(CXX is None, reason="no host C++ compiler")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "host_driver")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "structured_sparse_head_amd", "csrc", "host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def _run(driver, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env=env, timeout=120)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    out = res.stdout.splitlines()
    assert len(out) == len(lines)
    return out


def test_wythoff_and_modified_rows(driver):
    rows = list(range(-2, 2001)) + [1_200_000_000, 1_327_217_884, 1_327_217_885, 2 ** 31 - 1]
    out = _run(driver, [f"wythoff {i}" for i in rows] + [f"modified {i}" for i in rows])
    for i, line in zip(rows + rows, out):
        pass
    for k, i in enumerate(rows):
        rc, a, b = map(int, out[k].split())
        rcm, am, bm = map(int, out[len(rows) + k].split())
        if i < 1:
            assert rc == E_INVAL and rcm == E_INVAL
        elif i <= 2000:
            assert rc == OK and (a, b) == oracle.wythoff_row(i)
            assert rcm == OK and (am, bm) == oracle.wythoff_row_modified(i)
        else:
            assert rc == E_RANGE
            assert (rcm == OK and am == i - 1) or rcm == E_RANGE


def test_windows(driver):
    cases = [(H, lo, hi) for H in (1, 2, 3, 12, 16, 100)
             for lo, hi in ((1, 1), (5, 65), (49, 197), (1, 2 ** 31 - 1), (7, 8))]
    bad = [(0, 1, 2), (3, 0, 2), (3, 5, 4)]
    out = _run(driver, [f"windows {H} {lo} {hi}" for H, lo, hi in cases + bad])
    for (H, lo, hi), line in zip(cases, out):
        v = list(map(int, line.split()))
        assert v[0] == OK and v[1:] == oracle.window_sizes(H, lo, hi)
    for line in out[len(cases):]:
        assert int(line.split()[0]) == E_INVAL


def _offsets_line(H, N, cap, a, b, w):
    return " ".join(map(str, ["offsets", H, N, cap, *a, *b, *w]))


def test_offset_tables_bit_exact_and_two_call_sizing(driver):
    rng = np.random.default_rng(17)
    cases = []
    for _ in range(300):
        H = int(rng.integers(1, 20))
        N = int(rng.choice([1, 2, 3, 5, 17, 100, 1000, 70000, 2 ** 31 - 1]))
        a = [int(x) for x in rng.integers(0, 60, size=H)]
        b = [int(x) for x in rng.integers(1, 60, size=H)]
        w = [int(x) for x in rng.integers(1, min(N, 10 ** 9) + 1, size=H)]
        cases.append((H, N, a, b, w))
    lines = [_offsets_line(H, N, 64 * H, a, b, w) for H, N, a, b, w in cases]
    lines += [_offsets_line(H, N, 0, a, b, w) for H, N, a, b, w in cases[:50]]
    out = _run(driver, lines)
    for (H, N, a, b, w), line in zip(cases, out):
        left, right = line.split(";")
        v = list(map(int, left.split()))
        ptr, offs = oracle.offset_table(N, a, b, w)
        assert v[0] == OK and v[1:] == list(ptr)
        assert list(map(int, right.split())) == list(offs)
    for (H, N, a, b, w), line in zip(cases[:50], out[len(cases):]):
        v = list(map(int, line.split(";")[0].split()))
        ptr, offs = oracle.offset_table(N, a, b, w)
        assert v[0] == (OK if len(offs) == 0 else E_RANGE) and v[1:] == list(ptr)


def test_descriptor_error_paths(driver):
    good = "desc 2 3 65 64 1 1 4 6 2 7 10 65 65 65"
    lines = [good,
             "desc 0 3 65 64 1 1 4 6 2 7 10 65 65 65",      # B < 1
             "desc 2 3 0 64 1 1 4 6 2 7 10 65 65 65",       # N < 1
             "desc 2 3 65 32 1 1 4 6 2 7 10 65 65 65",      # d_h
             "desc 2 3 65 64 7 1 4 6 2 7 10 65 65 65",      # dtype
             "desc 2 3 65 64 1 -1 4 6 2 7 10 65 65 65",     # a < 0
             "desc 2 3 65 64 1 1 4 6 0 7 10 65 65 65",      # b < 1
             "desc 2 3 65 64 1 1 4 6 2 7 10 65 66 65",      # w > N
             "desc 2 3 65 64 1 1 4 6 2 7 10 0 65 65",       # w < 1
             "desc 1 129 65 64 1 " + " ".join(["1"] * 129 + ["2"] * 129 + ["65"] * 129),  # H > 128
             "desc 2147483647 128 2147483647 64 1 " + " ".join(["1"] * 128 + ["2"] * 128 + ["9"] * 128),
             ]
    out = [int(x) for x in _run(driver, lines)]
    assert out[0] == 2 * 3 * 65
    assert all(x == -1 for x in out[1:])


def test_table_error_paths(driver):
    lines = ["table 2 2 65 64 1 0 0 2 3 1 5 7",          # good: head 0 {1, 5}, head 1 {7}
             "table 2 2 65 64 1 1 0 2 3 1 5 7",          # good, class token
             "table 2 2 65 64 1 2 0 2 3 1 5 7",          # cls not 0/1
             "table 2 2 65 64 1 0 1 2 3 1 5 7",          # head_ptr[0] != 0
             "table 2 2 65 64 1 0 0 3 2 1 5 7",          # decreasing head_ptr
             "table 2 2 65 64 1 0 0 2 3 5 1 7",          # not ascending
             "table 2 2 65 64 1 0 0 2 3 1 65 7",         # distance >= N
             "table 2 2 65 64 1 0 0 2 3 -1 5 7",         # distance < 0
             "table 2 1 65 64 1 0 0 65 " + " ".join(map(str, range(65))),  # 65 > 64 distances
             ]
    out = [int(x) for x in _run(driver, lines)]
    assert out[0] == 2 * 2 * 65
    assert out[1] > 2 * 2 * 65
    assert all(x == -1 for x in out[2:])


def test_layout_error_paths(driver):
    B, H, N, D = 2, 3, 65, 64
    dense = f"{H * N * D} {N * D} {D}"

    def lay(bwd, dt=1, **over):
        names = ["q", "k", "v", "o", "dout", "dq", "dk", "dv"]
        parts = [over.get(n, dense) for n in names]
        return f"layouts {bwd} {B} {H} {N} {D} {dt} " + " ".join(parts)

    lines = [lay(0), lay(1), lay(0, q="0 0 64"), lay(0, o="0 4160 64"), lay(0, o="12480 0 64"),
             lay(1, dq="0 4160 64"), lay(1, dk="12480 0 64"), lay(0, q="-64 64 64"),
             lay(0, k="0 0 32"), lay(0, v="4 64 64"), lay(0, o=f"{(1 << 62) - 8} 64 64"),
             lay(1, dq="2 64 64", dt=1), lay(1, dv="0 1152921504606846976 1152921504606846976"),
             lay(0, o="12480 4160 128"), lay(1, o="-1 -1 -1")]
    out = [tuple(map(int, x.split())) for x in _run(driver, lines)]
    assert out[0] == (OK, 0) and out[1] == (OK, 0)       # dense
    assert out[2] == (OK, 1)                              # broadcast input
    assert all(o[0] == E_INVAL for o in out[3:13])
    assert out[13] == (OK, 1)                             # padded rows
    assert out[14] == (OK, 0)                             # the backward ignores o
