"""CPU oracle for Fibottention sparse attention -- test infrastructure only.

Imported solely by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  Independent of the HIP library: it
neither imports nor links anything from ``structured_sparse_head_amd``.
"""

from .fibottention import (  # noqa: F401
    backward,
    block_backward,
    block_forward,
    cls_support_mask,
    dense_backward,
    dense_forward,
    fib_offsets,
    fib_term,
    fib_successor,
    forward,
    offset_table,
    signed_offsets,
    support_mask,
    window_sizes,
    wythoff_row,
    wythoff_row_modified,
    wythoff_rows,
    zeckendorf,
)
