"""Content-adaptive block layout and its attention, in fp64 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages give: the Adaptive Sparse Transformer page ("Adapt or Perish:
新手入门指南 – Adaptive Sparse Transformer 核心原理与实战"), section on importance
evaluation, computes the attention scores of candidate positions and keeps
the highest r% per query (its code: top floor(L r) scores of each row, then
softmax over them and the product with V; r = 0.3 in the example).  The SQA
page ("Transformer计算效率优化：SQA稀疏注意力机制详解"), sections 3.1 and 5, stores
masks as 64x64 blocks and runs attention only on the non-zero blocks.

Reading taken: the selection is made per 64-token block, from the data, so
that the result is a block layout the block-sparse path can run:
* a block's representative is the sum of its 64 rows (the mean up to the
  positive factor 1/64, which changes no ranking): qs[i] = sum of q[64i + u]
  over u = 0..63, added in that order in fp64; ks[j] likewise from k;
* the score of block pair (i, j) is sum_d qs[i, d] * ks[j, d], each product
  rounded, then added in order d = 0..D-1, in fp64 (no fused multiply-add),
  so that any implementation doing the same operations gets the same bits;
* query block i keeps the keep = floor(nb r) (>= 1) key blocks of highest
  score, ties to the lower block index, listed ascending;
* attention is then the masked softmax of the usual definition over the kept
  blocks' tokens.
The layout differs per (batch, head), since it follows the data.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Tuple

import numpy as np

from .attention import _as_f64, masked_attention


def keep_blocks(num_blocks: int, ratio: float) -> int:
    """floor(nb * r), at least 1 and at most nb (the page's int(L * r) on blocks)."""
    return max(1, min(num_blocks, int(num_blocks * ratio)))


def block_sums(x: np.ndarray, block: int = 64) -> np.ndarray:
    """[L, D] -> [L/block, D]: rows of each block added in order, fp64."""
    x = np.asarray(x, dtype=np.float64)
    L, D = x.shape
    nb = L // block
    xb = x.reshape(nb, block, D)
    s = np.zeros((nb, D))
    for u in range(block):          # sequential over the block's rows
        s = s + xb[:, u, :]
    return s


def block_scores(qs: np.ndarray, ks: np.ndarray) -> np.ndarray:
    """[nb, D] x [nb, D] -> [nb, nb]: sum over d in order of the rounded products."""
    nb, D = qs.shape
    s = np.zeros((qs.shape[0], ks.shape[0]))
    for d in range(D):              # sequential over d; multiply, then add (no fusion)
        s = s + qs[:, d][:, None] * ks[:, d][None, :]
    return s


def select_blocks(scores: np.ndarray, keep: int) -> List[List[int]]:
    """Per row, the `keep` largest scores (ties to the lower index), ascending."""
    rows = []
    for i in range(scores.shape[0]):
        order = sorted(range(scores.shape[1]), key=lambda j: (-scores[i, j], j))
        rows.append(sorted(order[:keep]))
    return rows


def adaptive_rows(q, k, keep: int) -> List[List[List[List[int]]]]:
    """rows[b][h][i]: the kept key blocks of query block i, for every (b, h)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, L, D = q.shape
    return [[select_blocks(block_scores(block_sums(q[b, h]), block_sums(k[b, h])), keep) for h in range(H)]
            for b in range(B)]


def adaptive_attention_forward(q, k, v, keep: int, scale: float,
                               rows: Optional[List] = None,
                               pairs: Optional[Iterable[Tuple[int, int]]] = None,
                               ) -> Tuple[np.ndarray, np.ndarray, List]:
    """O [B, H, L, D], LSE [B, H, L] (NaN outside the selected (b, h) pairs) and the rows."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = q.shape
    nb = L // 64
    if rows is None:
        rows = adaptive_rows(q, k, keep)
    o = np.full((B, H, L, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]):
        bm = np.zeros((nb, nb), dtype=bool)
        for i, r in enumerate(rows[b][h]):
            bm[i, r] = True
        mask = np.repeat(np.repeat(bm, 64, axis=0), 64, axis=1)
        o[b, h], lse[b, h] = masked_attention(q[b, h], k[b, h], v[b, h], mask, scale)
    return o, lse, rows
