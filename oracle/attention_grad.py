"""Gradients of dense masked softmax attention in fp64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What is differentiated: the forward of ``oracle.attention`` -- the
SparseAttention formula of the Adaptive Sparse Transformer page ("Adapt or
Perish: 新手入门指南 – Adaptive Sparse Transformer 核心原理与实战"), softmax
of the scaled scores under the 0/1 mask, times V, with masked scores at
-inf.  The pages train these models (SQA page, "Transformer计算效率优化：SQA
稀疏注意力机制详解", sections 2.2 and 3.2 on training the sparse pattern and
mixed-precision training; BigBird page, "避坑指南" on mixed-precision training
and gradient checkpointing) but print no backward pass.  The reading taken:
the backward is the exact derivative of that forward with respect to Q, K
and V, for an upstream gradient dO of the output.  LSE is treated as a
statistic of the forward (no gradient flows into it).

With P the masked softmax of S = scale * Q K^T (row-wise over the allowed
keys) and O = P V, the chain rule gives, row by row:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))          (softmax Jacobian)
    dQ = scale * dS K
    dK = scale * dS^T Q

A row with no allowed key has P = 0 and contributes nothing.  The matrix
products are library primitives (numpy/BLAS), one step each.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .attention import _as_f64
from .layout import Layout


def masked_softmax(s: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax of s over the allowed entries; rows with none give 0."""
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    p = p / np.where(empty, 1.0, l)[:, None]
    p[empty] = 0.0
    return p


def masked_attention_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                          scale: float, do: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) of O = softmax(scale q k^T, masked) v for one head, given dO.

    q [n, D], k [m, D], v [m, D], mask [n, m] bool, do [n, D].  fp64.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p = masked_softmax(scale * (q @ k.T), mask)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, layout: Layout, scale: float,
                       valid_len: Optional[Sequence[int]] = None,
                       heads: Optional[Iterable[int]] = None,
                       batches: Optional[Iterable[int]] = None,
                       chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Block-sparse attention backward over [B, H, L, D] inputs by dense masking.

    Rows are taken ``chunk`` at a time: each chunk's dQ rows are its own, and
    its dK, dV contributions are summed over the chunks (the products above
    are sums over rows, so chunking does not change the definition).
    ``valid_len[b]`` masks keys s >= valid_len[b].  Returns (dQ, dK, dV)
    [B, H, L, D] in fp64 for the selected batches and heads (others NaN).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H, L, D = q.shape
    dq = np.full((B, H, L, D), np.nan)
    dk = np.full((B, H, L, D), np.nan)
    dv = np.full((B, H, L, D), np.nan)
    for b in (range(B) if batches is None else batches):
        vl = None if valid_len is None else int(valid_len[b])
        for h in (range(H) if heads is None else heads):
            dk[b, h] = 0.0
            dv[b, h] = 0.0
            for t0 in range(0, L, chunk):
                t = np.arange(t0, min(L, t0 + chunk))
                mask = layout.token_mask_rows(h, t, vl)
                gq, gk, gv = masked_attention_grad(q[b, h, t], k[b, h], v[b, h], mask, scale, do[b, h, t])
                dq[b, h, t] = gq
                dk[b, h] += gk
                dv[b, h] += gv
    return dq, dk, dv


def routed_attention_backward(q, k, v, do, routed_rows: np.ndarray, band_tokens: int, scale: float,
                              heads: Optional[Iterable[int]] = None,
                              batches: Optional[Iterable[int]] = None,
                              chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of the routed-query attention (SQA page, section 2.1; the
    forward is ``attention.routed_attention_forward``) by dense masking: row t
    sees every key if it is one of routed_rows[b, h], else the keys with
    |t - s| <= band_tokens.  Chunked over rows like ``attention_backward``.
    Returns (dQ, dK, dV) [B, H, L, D] in fp64 for the selected batches and
    heads (others NaN)."""
    from .attention import routed_token_mask_rows
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    routed_rows = np.asarray(routed_rows)
    B, H, L, D = q.shape
    dq = np.full((B, H, L, D), np.nan)
    dk = np.full((B, H, L, D), np.nan)
    dv = np.full((B, H, L, D), np.nan)
    for b in (range(B) if batches is None else batches):
        for h in (range(H) if heads is None else heads):
            dk[b, h] = 0.0
            dv[b, h] = 0.0
            for t0 in range(0, L, chunk):
                t = np.arange(t0, min(L, t0 + chunk))
                mask = routed_token_mask_rows(t, L, routed_rows[b, h], band_tokens)
                gq, gk, gv = masked_attention_grad(q[b, h, t], k[b, h], v[b, h], mask, scale, do[b, h, t])
                dq[b, h, t] = gq
                dk[b, h] += gk
                dv[b, h] += gv
    return dq, dk, dv

