"""Fibottention sparse multi-head attention for AMD MI355X (gfx950).

The compute path is the HIP library libfibatt.so (C ABI in include/fibatt.h);
this package only marshals arguments to it.
"""

from .fibatt import (  # noqa: F401
    BF16,
    E_HIP,
    E_INVAL,
    E_RANGE,
    E_UNSUPPORTED,
    EXPORTED,
    F32,
    LIB_PATH,
    FABRIC_OUT_BYTES,
    MAX_HEADS,
    OK,
    FibattError,
    Layout,
    Layouts,
    Fibottention,
    FibottentionFunction,
    FibottentionQKVFunction,
    FibottentionTable,
    backward,
    fabric_read,
    forward,
    hbm_stream,
    lib,
    offsets,
    time_next_call,
    windows,
    wythoff,
    wythoff_modified,
    wythoff_rows,
)
from .block import FibottentionAttention  # noqa: F401,E402
