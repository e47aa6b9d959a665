"""Seeded synthetic inputs for the five Fibottention attention workloads.

Shared by the oracle-side and HIP-side of the tests and by the benchmark.
This module only draws and casts random tensors; it holds none of the
method's arithmetic (no offsets, no Wythoff rows, no attention).  Head i of a
workload uses Wythoff row i (1-based); each side derives (a_i, b_i) itself.

Stand-ins: the Fibottention experiments run on CIFAR-10/100, Tiny-ImageNet
(ViT tokens) and action-recognition videos; no dataset is used here.  The
tensors below have the token counts and head shapes of those models, with
i.i.d. Gaussian entries (or a low-rank-peaked variant).

Recipe (numpy ``default_rng(seed)``, float32 draws, then one cast to the
workload dtype with round-to-nearest-even):

* draw order Q, K, V, dO with seed = workload number;
* "highres": U [B,H,N,8], W [B,H,8,d], G_Q, G_K, G_V, dO in that order;
  L = U W / sqrt(8); Q = 0.5 G_Q + L; K = 0.5 G_K + L; V = 0.5 G_V;
* "video": per-head windows w_i drawn with ``default_rng(1003).integers``
  uniformly from ceil(N/4) .. N inclusive.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    values: str         # "normal" or "lowrank"
    window: str         # "N" or "uniform_quarter"

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-vit B2 H3 N65 d64 fp32", 2, 3, 65, 64, "f32", "normal", "N"),
    2: Workload(2, "vit-b16-224 B64 H12 N197 d64 bf16", 64, 12, 197, 64, "bf16", "normal", "N"),
    3: Workload(3, "video-8x14x14 B16 H12 N1569 d64 bf16", 16, 12, 1569, 64, "bf16", "normal",
                "uniform_quarter"),
    4: Workload(4, "highres-64x64 B4 H16 N4097 d64 bf16", 4, 16, 4097, 64, "bf16", "lowrank", "N"),
    5: Workload(5, "long-1d B1 H16 N65536 d128 bf16", 1, 16, 65536, 128, "bf16", "normal", "N"),
}


def windows(wl: Workload) -> np.ndarray:
    """Per-head window w_i (int32[H])."""
    if wl.window == "N":
        return np.full(wl.H, wl.N, dtype=np.int32)
    lo = -(-wl.N // 4)
    rng = np.random.default_rng(1000 + wl.number)
    return rng.integers(lo, wl.N + 1, size=wl.H).astype(np.int32)


def _cast(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def make_inputs(wl: Workload, seed: Optional[int] = None, with_grad_out: bool = True,
                B: Optional[int] = None, H: Optional[int] = None,
                N: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Q, K, V (and dO) as contiguous CPU tensors [B, H, N, d] in the workload dtype.

    B, H, N may be overridden for reduced test cases (same distribution).
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    N = wl.N if N is None else N
    d = wl.d
    rng = np.random.default_rng(wl.number if seed is None else seed)
    shape = (B, H, N, d)
    out = {}
    if wl.values == "normal":
        for name in ("q", "k", "v") + (("do",) if with_grad_out else ()):
            out[name] = _cast(rng.standard_normal(shape, dtype=np.float32), wl.torch_dtype)
    elif wl.values == "lowrank":
        r = 8
        U = rng.standard_normal((B, H, N, r), dtype=np.float32)
        W = rng.standard_normal((B, H, r, d), dtype=np.float32)
        L = np.matmul(U, W) / np.float32(math.sqrt(r))
        g = {n: rng.standard_normal(shape, dtype=np.float32) for n in ("q", "k", "v")}
        out["q"] = _cast(0.5 * g["q"] + L, wl.torch_dtype)
        out["k"] = _cast(0.5 * g["k"] + L, wl.torch_dtype)
        out["v"] = _cast(0.5 * g["v"], wl.torch_dtype)
        if with_grad_out:
            out["do"] = _cast(rng.standard_normal(shape, dtype=np.float32), wl.torch_dtype)
    else:
        raise ValueError(wl.values)
    return out


def random_case(seed: int, B: int, H: int, N: int, d: int, dtype: torch.dtype,
                with_grad_out: bool = True) -> Dict[str, torch.Tensor]:
    """i.i.d. N(0,1) tensors of an arbitrary shape (edge-case tests)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    names = ("q", "k", "v") + (("do",) if with_grad_out else ())
    return {n: _cast(rng.standard_normal(shape, dtype=np.float32), dtype) for n in names}
