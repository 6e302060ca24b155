"""The attention layer around the block-sparse attention, in fp64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Follows the primer page ("BERT稀疏注意力机制入门指南：原理、实现与性能优化",
section PyTorch 实现基础稀疏注意力), the SparseAttention module: one linear map
x -> qkv of width 3C (weight [3C, C] and bias, as nn.Linear), the width-3C
row read as (3, H, C/H) -- q, k, v, then heads, then the head's features --
attention per head, the heads concatenated back to width C in head order, and
the output linear map (weight [C, C] and bias).  The attention itself is
``oracle.attention`` (block layout, key padding, the scale as an argument; the
page divides by sqrt(C), the workloads here by sqrt(C/H)).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import _as_f64, attention_forward
from .layout import Layout


def layer_forward(x, w_qkv, b_qkv, w_proj, b_proj, layout: Layout, num_heads: int, scale: float,
                  valid_len: Optional[Sequence[int]] = None) -> np.ndarray:
    """out [B, L, C] = proj(attention(split(x @ w_qkv^T + b_qkv))) in fp64."""
    x, w_qkv, b_qkv, w_proj, b_proj = (_as_f64(t) for t in (x, w_qkv, b_qkv, w_proj, b_proj))
    B, L, C = x.shape
    H = num_heads
    D = C // H
    qkv = x @ w_qkv.T + b_qkv                                  # [B, L, 3C]
    qkv = qkv.reshape(B, L, 3, H, D)
    q, k, v = (np.ascontiguousarray(qkv[:, :, s].transpose(0, 2, 1, 3)) for s in range(3))   # [B, H, L, D]
    o, _ = attention_forward(q, k, v, layout, scale, valid_len=valid_len)
    o = o.transpose(0, 2, 1, 3).reshape(B, L, C)               # heads concatenated in order
    return o @ w_proj.T + b_proj
