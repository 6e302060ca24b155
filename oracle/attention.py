"""Dense masked softmax attention in fp64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Definition followed: Adaptive Sparse Transformer page ("Adapt or Perish:
新手入门指南 – Adaptive Sparse Transformer 核心原理与实战"), the SparseAttention
formula -- softmax of the scaled scores Q K^T / sqrt(d_k) under a 0/1 mask M,
times V.  The formula writes the mask as an elementwise product; the code on
the primer page ("BERT稀疏注意力机制入门指南：原理、实现与性能优化", PyTorch 实现基础稀疏注意力)
and on the multi-head page ("BERT多头注意力机制深度解析：如何优化长文本处理性能")
fills masked scores with a very negative number before the softmax.  The
reading taken: masked scores are -inf, i.e. masked keys get weight exactly 0.
With at least one allowed key per row this equals the pages' finite fill in
fp64; a row with no allowed key returns O = 0 and LSE = -inf.

The patterns are combined with ONE softmax over the union mask (the formula
has a single M); the BigBird page's code sums three separately normalised
attentions, which is not followed.

LSE is the natural-log log-sum-exp of the scaled, masked scores of a row
(scale included), the statistic a backward pass needs.

Inputs are promoted to fp64 exactly (bf16 and fp32 values are fp64 values).
The matrix product is a library primitive (numpy/BLAS) used as one step.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .layout import Layout


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * q k^T, masked) v for one head.

    q [n, D], k [m, D], v [m, D], mask [n, m] bool.  Returns (O [n, D], LSE [n]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])          # masked entries: exp(-inf) = 0
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    o = (p @ v) / l_safe[:, None]
    o[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def _as_f64(x) -> np.ndarray:
    """Exact promotion of a torch tensor (fp32/bf16) or array to fp64 numpy."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def attention_forward(q, k, v, layout: Layout, scale: float,
                      valid_len: Optional[Sequence[int]] = None,
                      heads: Optional[Iterable[int]] = None,
                      batches: Optional[Iterable[int]] = None,
                      chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Block-sparse attention forward over [B, H, L, D] inputs by dense masking.

    Rows are processed ``chunk`` at a time to bound memory; chunking does not
    change the definition.  ``valid_len[b]`` masks keys s >= valid_len[b].
    Returns (O [B, H, L, D], LSE [B, H, L]) in fp64 for the selected batches
    and heads (others left NaN).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = q.shape
    o = np.full((B, H, L, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in (range(B) if batches is None else batches):
        vl = None if valid_len is None else int(valid_len[b])
        for h in (range(H) if heads is None else heads):
            for t0 in range(0, L, chunk):
                t = np.arange(t0, min(L, t0 + chunk))
                mask = layout.token_mask_rows(h, t, vl)
                o[b, h, t], lse[b, h, t] = masked_attention(q[b, h, t], k[b, h], v[b, h], mask, scale)
    return o, lse


def attention_rows(q, k, v, layout: Layout, scale: float, rows: Sequence[Tuple[int, int, int]],
                   valid_len: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition evaluated only at the given (b, h, t) rows, one by one."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    D = q.shape[-1]
    o = np.empty((len(rows), D))
    lse = np.empty(len(rows))
    for n, (b, h, t) in enumerate(rows):
        vl = None if valid_len is None else int(valid_len[b])
        mask = layout.token_mask_rows(h, np.array([t]), vl)
        o[n], lse[n] = (x[0] for x in masked_attention(q[b, h, t][None], k[b, h], v[b, h], mask, scale))
    return o, lse


def routed_token_mask_rows(t_rows: np.ndarray, seq_len: int, routed: Sequence[int],
                           band_tokens: int) -> np.ndarray:
    """Mask of the routed-query variant for one head: row t sees every key if t is
    routed, else only keys with |t - s| <= band (SQA page, section 2.1)."""
    t_rows = np.asarray(t_rows, dtype=np.int64)
    s = np.arange(seq_len)
    band = np.abs(t_rows[:, None] - s[None, :]) <= band_tokens
    is_routed = np.isin(t_rows, np.asarray(routed, dtype=np.int64))
    return band | is_routed[:, None]


def routed_attention_forward(q, k, v, routed_rows: np.ndarray, band_tokens: int, scale: float,
                             heads: Optional[Iterable[int]] = None,
                             rows: Optional[Sequence[Tuple[int, int, int]]] = None,
                             chunk: int = 1024):
    """Routed-query attention.  ``routed_rows`` [B, H, k].

    With ``rows`` given, evaluates only those (b, h, t) rows and returns
    (O [n, D], LSE [n]); otherwise returns full (O [B,H,L,D], LSE [B,H,L]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = q.shape
    routed_rows = np.asarray(routed_rows)
    if rows is not None:
        o = np.empty((len(rows), D))
        lse = np.empty(len(rows))
        for n, (b, h, t) in enumerate(rows):
            mask = routed_token_mask_rows(np.array([t]), L, routed_rows[b, h], band_tokens)
            oo, ll = masked_attention(q[b, h, t][None], k[b, h], v[b, h], mask, scale)
            o[n], lse[n] = oo[0], ll[0]
        return o, lse
    o = np.full((B, H, L, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            for t0 in range(0, L, chunk):
                t = np.arange(t0, min(L, t0 + chunk))
                mask = routed_token_mask_rows(t, L, routed_rows[b, h], band_tokens)
                o[b, h, t], lse[b, h, t] = masked_attention(q[b, h, t], k[b, h], v[b, h], mask, scale)
    return o, lse
