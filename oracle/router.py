"""Routed-query selection (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

SQA page ("Transformer计算效率优化：SQA稀疏注意力机制详解"), section 2.1: a learned
router scores every query with a single linear projection (width -> 1) and
keeps the top-k queries, which then attend globally; section 3.2 keeps the
router in FP32 while the model runs in FP16.

Readings taken:
* No bias; the projection vector w is an input (fixed by a seed).
* score[b, h, t] = sum over d of q[b,h,t,d] * w[d], evaluated in fp64 as a
  left-to-right sum in d.  A bf16 x fp32 product has at most 32 significant
  bits, so every product is exact in fp64 and only the additions round --
  a fused multiply-add and a multiply-then-add give the same bits, and any
  implementation that sums in the same order reproduces the score exactly.
  This is at least the FP32 precision the page asks for.
* top-k per (b, h): order rows by (score descending, index ascending) --
  ties go to the lower index -- keep the first k, report them ascending.
"""
from __future__ import annotations

import numpy as np


def router_scores(q, w) -> np.ndarray:
    """Exact-order fp64 scores: [B, H, L] from q [B, H, L, D] and w [D]."""
    from .attention import _as_f64
    q = _as_f64(q)
    w = _as_f64(w)
    acc = np.zeros(q.shape[:-1], dtype=np.float64)
    for d in range(q.shape[-1]):
        acc = acc + q[..., d] * w[d]
    return acc


def topk_rows(scores: np.ndarray, k: int) -> np.ndarray:
    """[B, H, k] int32: the k best rows per (b, h) by (-score, index), ascending."""
    B, H, L = scores.shape
    out = np.empty((B, H, k), dtype=np.int32)
    idx = np.arange(L)
    for b in range(B):
        for h in range(H):
            order = np.lexsort((idx, -scores[b, h]))   # last key is primary
            out[b, h] = np.sort(order[:k])
    return out
