"""Build configuration (CPU only): the per-file compile flags name files that
are built, and they enter the source hash that gates the committed traffic
counters in the benchmark line."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from structured_sparse_head_amd import build  # noqa: E402


def test_file_flags_name_built_sources():
    assert set(build.FILE_FLAGS) <= set(build.SOURCES)
    for src, flags in build.FILE_FLAGS.items():
        assert os.path.exists(os.path.join(build.CSRC, src))
        assert flags and len(flags) % 2 == 0 and all(f == "-mllvm" for f in flags[::2])


def test_file_flags_enter_the_source_hash(monkeypatch):
    import bench
    h0 = bench.source_hash("bwd_slab_bf16_kernel")
    t0 = bench.source_hash("bwd_dq_tile_kernel")
    flags = dict(build.FILE_FLAGS)
    flags["bwd_slab_bf16.hip"] = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
    monkeypatch.setattr(build, "FILE_FLAGS", flags)
    assert bench.source_hash("bwd_slab_bf16_kernel") != h0
    assert bench.source_hash("bwd_dq_tile_kernel") == t0  # other files unaffected
