"""One Fibottention multi-head self-attention layer (README Algorithm 3).

X [B, N, c] -> Q_i = X W_i^Q, K_i = X W_i^K, V_i = X W_i^V for heads
i = 1..h (d_h = c / h) -> Z_i = sparse Fibottention attention of head i ->
O = concat(Z_1..Z_h) W^Z.  The four projections are plain dense GEMMs and
run through torch (hipBLASLt on MFMA); the sparse core is the HIP library
behind ``fibatt_fwd`` / ``fibatt_bwd`` (or the class-token entry points), with
its 1/sqrt(d_h) score scale.  The kernels read Q, K and V as strided views of
the fused projection's output and write O straight into the [B, N, h, d_h]
order the output projection reads (``FibottentionQKVFunction``), so the
layer makes no head split or merge copies.  Gradients of the projections come
from torch autograd around that function.

Heads use Wythoff rows 1..h (or README Algorithm 2's modified pairs) and the
windows interpolated between w_min and w_max (Fibottention paper, method
section); with no windows given every head sees the whole sequence.
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from .fibatt import FibottentionQKVFunction, windows, wythoff_rows


class FibottentionAttention(torch.nn.Module):
    """Parameters: ``w_qkv`` [c, 3c] = [W^Q | W^K | W^V] (head i owns columns
    i*d_h .. (i+1)*d_h of each third) and ``w_z`` [c, c]; no biases, as in
    the README's Algorithm 3."""

    def __init__(self, dim: int, heads: int, n_tokens: int, w_min: Optional[int] = None,
                 w_max: Optional[int] = None, modified: bool = False, cls: bool = False,
                 device=None, dtype=torch.bfloat16):
        super().__init__()
        if dim % heads:
            raise ValueError("dim must be a multiple of heads")
        self.dim, self.heads, self.n_tokens = dim, heads, n_tokens
        self.d_h = dim // heads
        self.cls = cls
        w_max = n_tokens if w_max is None else w_max
        w_min = w_max if w_min is None else w_min
        self.a, self.b = wythoff_rows(heads, modified=modified)
        self.w = windows(heads, w_min, w_max)
        self.w_qkv = torch.nn.Parameter(torch.empty(dim, 3 * dim, device=device, dtype=dtype))
        self.w_z = torch.nn.Parameter(torch.empty(dim, dim, device=device, dtype=dtype))
        self.reset_parameters()

    def reset_parameters(self, generator: Optional[torch.Generator] = None) -> None:
        std = 1.0 / math.sqrt(self.dim)
        with torch.no_grad():
            for p in (self.w_qkv, self.w_z):
                p.copy_(torch.randn(p.shape, generator=generator, dtype=torch.float32) * std)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        B, N, c = x.shape
        if N != self.n_tokens or c != self.dim:
            raise ValueError(f"expected [B, {self.n_tokens}, {self.dim}], got {tuple(x.shape)}")
        qkv = torch.mm(x.reshape(B * N, c), self.w_qkv).view(B, N, 3, self.heads, self.d_h)
        z = FibottentionQKVFunction.apply(qkv, self.a, self.b, self.w, self.cls)
        return torch.mm(z.view(B * N, c), self.w_z).view(B, N, c)
