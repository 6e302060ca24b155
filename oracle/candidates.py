"""Candidate-list attention (oracle): the Adaptive page's candidate generator
followed by its importance evaluation.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Adaptive Sparse Transformer page ("Adapt or Perish: 新手入门指南 – Adaptive
Sparse Transformer 核心原理与实战"), the two parts of its dynamic mask:
* the candidate generator, a light CNN -- a Conv1d from the model width to
  k = 32 channels, kernel 3, padding 1 -- that predicts k relevant
  positions for every query from the hidden states x [B, L, C];
* the importance evaluation, which scores the candidate positions and keeps
  the best r% (r = 0.3), and the SparseAttention formula over what is kept.

Readings taken:
* The k outputs of the convolution at token t are k key positions, in
  tokens from the start of the sequence: position = the output rounded to
  the nearest integer (ties to even), clamped to [0, L - 1]; a NaN output
  gives 0.  Positions that coincide count once (the candidate set).
* The convolution is PyTorch's Conv1d: y[b, t, j] = bias[j] + sum over
  taps u = 0, 1, 2 and channels c of W[j, c, u] * x[b, t + u - 1, c], with
  zeros outside the sequence.  The rounding makes the position an integer
  decision taken from floating point, so the sum has a fixed evaluation:
  fp64, starting from bias[j], adding the products for u = 0, 1, 2 in turn
  and within a tap for c = 0 .. C - 1.  A bf16 x fp32 product has at most
  32 significant bits and is exact in fp64, so only the additions round.
  Taps outside the sequence add nothing.
* The importance evaluation keeps floor(k r) of the candidates per (batch,
  head, query), ranked by the in-order fp32 score q.k of the top-keep
  oracle (``topr.ranking_scores``), ties to the lower position; a query with
  fewer distinct candidates keeps them all.
* The attention over the kept keys is the SparseAttention formula with
  scale 1/sqrt(D) (M = 1 on the kept keys), in fp64 (``masked_attention``).
* The generator's weights are inputs (the page's are trained; seeded ones
  stand in for them).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .attention import _as_f64, masked_attention
from .topr import _as_f32, ranking_scores


def conv_outputs(x, w, bias) -> np.ndarray:
    """fp64 [B, L, k]: the convolution in the fixed order above.
    x [B, L, C] (bf16 data), w [k, C, 3] fp32, bias [k] fp32."""
    x = _as_f64(x)
    w = np.asarray(w, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    B, L, C = x.shape
    k = w.shape[0]
    acc = np.broadcast_to(bias, (B, L, k)).copy()
    for u in range(3):
        # x[b, t + u - 1, :], zero outside the sequence
        xs = np.zeros_like(x)
        lo, hi = max(0, 1 - u), min(L, L + 1 - u)
        xs[:, lo:hi] = x[:, lo + u - 1:hi + u - 1]
        for c in range(C):
            acc = acc + xs[:, :, c, None] * w[None, None, :, c, u]
    return acc


def positions_from_outputs(y: np.ndarray, seq_len: int) -> np.ndarray:
    """int32 positions: round half to even, clamp to [0, L - 1], NaN -> 0."""
    p = np.rint(np.nan_to_num(y, nan=0.0, posinf=float(seq_len), neginf=-1.0))
    return np.clip(p, 0, seq_len - 1).astype(np.int32)


def candidate_positions(x, w, bias) -> np.ndarray:
    """[B, L, k] int32 candidate positions of every query."""
    return positions_from_outputs(conv_outputs(x, w, bias), _as_f64(x).shape[1])


def kept_candidates(q_row, k_rows_all, positions_row, keep: int) -> np.ndarray:
    """Ascending kept key positions of one query: the distinct candidates ranked
    by (fp32 in-order score descending, position ascending), the first `keep`."""
    cand = np.unique(np.asarray(positions_row, dtype=np.int64))
    s = ranking_scores(np.asarray(q_row)[None], np.asarray(k_rows_all)[cand])[0]
    order = np.lexsort((cand, -s.astype(np.float64)))
    return np.sort(cand[order[:keep]])


def kept_mask(q, k, positions, keep: int, heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """Boolean [B, H, L, L] (listed heads; others all False): key s kept by query t."""
    q32, k32 = _as_f32(q), _as_f32(k)
    positions = np.asarray(positions)
    B, H, L, _ = q32.shape
    out = np.zeros((B, H, L, L), dtype=bool)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            for t in range(L):
                out[b, h, t, kept_candidates(q32[b, h, t], k32[b, h], positions[b, t], keep)] = True
    return out


def candidate_attention_forward(q, k, v, positions, keep: int, scale: float,
                                heads: Optional[Iterable[int]] = None,
                                rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Attention of every query over its kept candidates.  With ``rows``, only
    those (b, h, t) (returns O [n, D], LSE [n]); otherwise O [B, H, L, D] and
    LSE [B, H, L] for the listed heads (NaN elsewhere)."""
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    q32, k32 = _as_f32(q), _as_f32(k)
    positions = np.asarray(positions)
    B, H, L, D = qf.shape
    if rows is not None:
        o = np.empty((len(rows), D))
        lse = np.empty(len(rows))
        for n, (b, h, t) in enumerate(rows):
            m = np.zeros((1, L), dtype=bool)
            m[0, kept_candidates(q32[b, h, t], k32[b, h], positions[b, t], keep)] = True
            oo, ll = masked_attention(qf[b, h, t][None], kf[b, h], vf[b, h], m, scale)
            o[n], lse[n] = oo[0], ll[0]
        return o, lse
    o = np.full((B, H, L, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            m = np.zeros((L, L), dtype=bool)
            for t in range(L):
                m[t, kept_candidates(q32[b, h, t], k32[b, h], positions[b, t], keep)] = True
            o[b, h], lse[b, h] = masked_attention(qf[b, h], kf[b, h], vf[b, h], m, scale)
    return o, lse
