"""Pins for the content-adaptive block layout oracle (CPU only).

Checked against exact rational arithmetic, a brute-force statement of the
top-k rule, the max/min separation the selection must satisfy, and the
dense special case (keep every block) against torch's fp64 attention.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import adaptive as OD


def _bf16_values(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).to(torch.float64).numpy()


def test_keep_blocks_is_the_pages_floor():
    assert OD.keep_blocks(128, 0.3) == 38     # int(128 * 0.3) = int(38.4)
    assert OD.keep_blocks(32, 0.3) == 9
    assert OD.keep_blocks(4, 0.1) == 1        # at least one block
    assert OD.keep_blocks(10, 1.0) == 10


def test_block_sums_are_exact_sums():
    x = _bf16_values((256, 8), 1)
    s = OD.block_sums(x)
    for i in range(4):
        for d in range(8):
            exact = sum(Fraction(float(v)) for v in x[64 * i:64 * i + 64, d])
            assert Fraction(float(s[i, d])) == exact


def test_block_scores_exact_on_integers():
    g = np.random.default_rng(2)
    qs = g.integers(-50, 50, size=(6, 16)).astype(np.float64)
    ks = g.integers(-50, 50, size=(7, 16)).astype(np.float64)
    s = OD.block_scores(qs, ks)
    want = [[sum(int(qs[i, d]) * int(ks[j, d]) for d in range(16)) for j in range(7)] for i in range(6)]
    assert s.tolist() == want


def test_block_scores_close_to_exact_rational():
    qs = OD.block_sums(_bf16_values((512, 64), 3))
    ks = OD.block_sums(_bf16_values((512, 64), 4))
    s = OD.block_scores(qs, ks)
    for i in range(8):
        for j in range(8):
            exact = sum(Fraction(float(qs[i, d])) * Fraction(float(ks[j, d])) for d in range(64))
            bound = 64 * 2.0 ** -52 * float(sum(abs(Fraction(float(qs[i, d])) * Fraction(float(ks[j, d])))
                                               for d in range(64)))
            assert abs(Fraction(float(s[i, j])) - exact) <= Fraction(bound)


def test_selection_brute_force_and_ties():
    g = np.random.default_rng(5)
    s = g.normal(size=(20, 20))
    s[3, 7] = s[3, 2] = s[3, 11] = 5.0          # three-way tie at the top of row 3
    s[4, :] = 0.0                               # a row of equal scores
    for keep in (1, 2, 5, 20):
        rows = OD.select_blocks(s, keep)
        for i in range(20):
            chosen = [j for j in range(20)
                      if sum(1 for jj in range(20) if s[i, jj] > s[i, j] or (s[i, jj] == s[i, j] and jj < j)) < keep]
            assert rows[i] == chosen
            assert len(rows[i]) == keep
            if keep < 20:
                rest = [j for j in range(20) if j not in rows[i]]
                assert min(s[i, rows[i]]) >= max(s[i, rest])
    assert OD.select_blocks(s, 2)[3] == [2, 7]
    assert OD.select_blocks(s, 3)[4] == [0, 1, 2]


def test_keep_everything_is_dense_attention():
    B, H, L, D = 1, 2, 256, 32
    q = torch.from_numpy(_bf16_values((B, H, L, D), 6))
    k = torch.from_numpy(_bf16_values((B, H, L, D), 7))
    v = torch.from_numpy(_bf16_values((B, H, L, D), 8))
    scale = D ** -0.5
    o, lse, rows = OD.adaptive_attention_forward(q, k, v, 4, scale)
    assert all(r == [0, 1, 2, 3] for rb in rows for rh in rb for r in rh)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale).numpy()
    assert np.abs(o - ref).max() < 1e-12
    ref_lse = torch.logsumexp(scale * q @ k.transpose(-1, -2), dim=-1).numpy()
    assert np.abs(lse - ref_lse).max() < 1e-12


def test_selected_blocks_follow_the_data():
    # a key block made to align with every query block is chosen by every row
    B, H, L, D = 1, 1, 512, 16
    c = np.sign(_bf16_values((D,), 11))
    q = c[None, None, None, :] + _bf16_values((B, H, L, D), 9, scale=0.1)
    k = _bf16_values((B, H, L, D), 10, scale=0.01)
    k[0, 0, 64 * 5:64 * 6, :] = 0.5 * c[None, :]
    rows = OD.adaptive_rows(q, k, 1)
    assert all(r == [5] for r in rows[0][0])
