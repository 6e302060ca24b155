"""Per-query top-keep attention (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Adaptive Sparse Transformer page ("Adapt or Perish: 新手入门指南 – Adaptive
Sparse Transformer 核心原理与实战"), its importance-evaluation step: every query
scores the keys, keeps the ⌊L·r⌋ highest (its code: r = 0.3), and attends to
those alone -- the SparseAttention formula with M the indicator of the kept
keys.

Readings taken:
* The printed code keeps only the top-k score *values* and multiplies their
  softmax by V, which does not match V's L rows.  The plain reading: keep the
  top ``keep`` keys of each query, set M = 1 there and 0 elsewhere, and apply
  the SparseAttention formula (softmax of scale · q·k over the kept keys,
  times their V rows).
* scale = 1/sqrt(D), from the SparseAttention formula (the code omits it;
  a positive scale does not change which keys rank highest).
* ``keep`` is passed as an integer (keep = ⌊L·r⌋; r = 0.3 gives ⌊0.3 L⌋).
* Ranking precision: the rank decides an integer, so it is taken on a score
  with a fixed evaluation: q·k in fp32, products added in order of d,
  starting from +0.  Every bf16 × bf16 product is exact in fp32 (8 + 8
  significant bits), so each step rounds only the addition and the score is
  reproducible bit for bit by any code that adds in the same order, fused or
  not.  Keys rank by (score descending, key index ascending): ties go to the
  lower index.  NaN scores (from NaN or infinite inputs) rank unspecified.
* The attention itself is evaluated in fp64 from the inputs (``masked_attention``),
  like every other attention of this oracle; only the choice of keys uses
  the fp32 ranking score.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .attention import _as_f64, masked_attention


def _as_f32(x) -> np.ndarray:
    """Exact promotion of bf16 (or fp32) data to fp32 numpy."""
    return _as_f64(x).astype(np.float32)


def ranking_scores(q, k) -> np.ndarray:
    """fp32 ranking scores [..., Lq, Lk]: sum over d of q[..., t, d] * k[..., s, d],
    added in order of d from +0, each product rounded to fp32 first (exact for bf16 data)."""
    q = _as_f32(q)
    k = _as_f32(k)
    acc = np.zeros(q.shape[:-1] + (k.shape[-2],), dtype=np.float32)
    for d in range(q.shape[-1]):
        prod = (q[..., :, None, d] * k[..., None, :, d]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    return acc


def kept_keys(scores_row: np.ndarray, keep: int) -> np.ndarray:
    """Ascending indices of the ``keep`` best keys of one row: (score desc, index asc)."""
    idx = np.arange(scores_row.shape[0])
    order = np.lexsort((idx, -scores_row.astype(np.float64)))
    return np.sort(order[:keep])


def topr_mask(q, k, keep: int, heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """Boolean [B, H, Lq, Lk] (or only the listed heads; others all False): key s kept by query t."""
    q = _as_f32(q)
    k = _as_f32(k)
    B, H, Lq, _ = q.shape
    out = np.zeros((B, H, Lq, k.shape[2]), dtype=bool)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            s = ranking_scores(q[b, h], k[b, h])
            for t in range(Lq):
                out[b, h, t, kept_keys(s[t], keep)] = True
    return out


def topr_attention_forward(q, k, v, keep: int, scale: float,
                           heads: Optional[Iterable[int]] = None,
                           rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Attention of every query over its ``keep`` top-ranked keys.

    With ``rows`` given, evaluates only those (b, h, t) rows and returns
    (O [n, D], LSE [n]); otherwise returns (O [B,H,L,D], LSE [B,H,L]) for the
    listed heads (NaN elsewhere)."""
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = qf.shape
    if rows is not None:
        o = np.empty((len(rows), D))
        lse = np.empty(len(rows))
        for n, (b, h, t) in enumerate(rows):
            s = ranking_scores(_as_f32(q)[b, h, t][None], _as_f32(k)[b, h])[0]
            m = np.zeros((1, L), dtype=bool)
            m[0, kept_keys(s, keep)] = True
            oo, ll = masked_attention(qf[b, h, t][None], kf[b, h], vf[b, h], m, scale)
            o[n], lse[n] = oo[0], ll[0]
        return o, lse
    o = np.full((B, H, L, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    q32, k32 = _as_f32(q), _as_f32(k)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            s = ranking_scores(q32[b, h], k32[b, h])
            m = np.zeros((L, L), dtype=bool)
            for t in range(L):
                m[t, kept_keys(s[t], keep)] = True
            o[b, h], lse[b, h] = masked_attention(qf[b, h], kf[b, h], vf[b, h], m, scale)
    return o, lse
