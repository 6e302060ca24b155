"""Pins for the oracle's token-granular pattern (CPU only).

The pattern is the block rule on 1-token blocks (already pinned by
test_oracle_layout.py); what is new here is checked against the page's own
global-token expression (torch.linspace(...).long()), exact rational
arithmetic, a hand-derived count, and closed-form row sizes computed
independently of the row construction.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import layout as OL


@pytest.mark.parametrize("L,n", [(8192, 8), (8192, 410), (8192, 819), (2048, 8), (2048, 103), (1024, 3),
                                 (4096, 205), (16384, 8)])
def test_global_tokens_equal_the_pages_linspace(L, n):
    # BigBird page code: torch.linspace(0, seq_len - 1, num_global).long()
    assert OL.linspace_tokens(L, n) == torch.linspace(0, L - 1, n).long().tolist()


@pytest.mark.parametrize("L,n", [(512, 64), (1024, 64), (100, 7), (8191, 13)])
def test_global_tokens_are_exact_floors(L, n):
    got = OL.linspace_tokens(L, n)
    want = [int(Fraction(i * (L - 1), n - 1)) for i in range(n)]   # int() of a positive Fraction floors
    assert got == want
    assert got[0] == 0 and got[-1] == L - 1
    assert len(set(got)) == n
    # float32 rounding moves at most one unit away from the exact value
    tl = torch.linspace(0, L - 1, n).long().tolist()
    assert max(abs(a - b) for a, b in zip(tl, got)) <= 1


def test_degenerate_global_counts():
    assert OL.linspace_tokens(100, 0) == []
    assert OL.linspace_tokens(100, 1) == [0]
    assert OL.linspace_tokens(100, 2) == [0, 99]


def test_rows_equal_the_block_rule_on_one_token_blocks():
    g = np.random.default_rng(5)
    for _ in range(6):
        L = int(g.integers(8, 200))
        w = int(g.integers(0, 6))
        ng = int(g.integers(0, 5))
        r = int(g.integers(0, 6))
        seed = int(g.integers(0, 2**63))
        tl = OL.make_token_layout(2, L, min(w, L - 1), ng, r, seed)
        bl = OL.make_layout(2, L, 1, 2 * min(w, L - 1) + 1, tl.global_tokens, r, seed)
        for h in range(2):
            for t in range(L):
                assert tl.row(h, t) == bl.rows[h][t]


def _closed_form_row_sizes(L, w, G, r):
    """|row t| from interval arithmetic alone: L for a global t, else
    |band| + |G outside the band| + min(r, L - |band U G|)."""
    t = np.arange(L)
    lo = np.maximum(0, t - w)
    hi = np.minimum(L - 1, t + w)
    band = hi - lo + 1
    Ga = np.asarray(G, dtype=np.int64)
    g_in = ((Ga[None, :] >= lo[:, None]) & (Ga[None, :] <= hi[:, None])).sum(axis=1) if len(G) else 0 * t
    e = band + len(G) - g_in
    size = e + np.minimum(r, L - e)
    size[np.isin(t, Ga)] = L
    return size


@pytest.mark.parametrize("L,w,ng,r,seed", [(16, 1, 2, 2, 0), (300, 7, 5, 4, 3), (2048, 64, 8, 8, 11),
                                           (1000, 20, 50, 8, 2), (64, 40, 3, 100, 9)])
def test_row_sizes_match_closed_form(L, w, ng, r, seed):
    tl = OL.make_token_layout(1, L, w, ng, r, seed)
    sizes = _closed_form_row_sizes(L, w, tl.global_tokens, r)
    G = set(tl.global_tokens)
    for t in range(L):
        row = tl.row(0, t)
        assert len(row) == sizes[t], t
        assert row == sorted(set(row))
        assert G <= set(row)
        assert set(range(max(0, t - w), min(L - 1, t + w) + 1)) <= set(row)
        links = tl.random_links(0, t)
        assert all(abs(s - t) > w and s not in G for s in links)


def test_hand_derived_count():
    # tests/golden/token_layout_nnz.txt: L=16, w=1, 2 global tokens {0, 15}, r=2
    rows = {r[0]: int(r[1]) for r in read_golden("token_layout_nnz.txt")}
    tl = OL.make_token_layout(1, 16, 1, 2, 2, 123)
    assert tl.global_tokens == [0, 15]
    assert sum(len(tl.row(0, t)) for t in range(16)) == rows["L16-w1-g2-r2"]


def test_token_mask_rows():
    tl = OL.make_token_layout(2, 96, 3, 4, 2, 77)
    t = np.array([0, 5, 31, 32, 95])
    m = tl.token_mask_rows(1, t)
    for n, tt in enumerate(t):
        assert np.flatnonzero(m[n]).tolist() == tl.row(1, int(tt))
    m2 = tl.token_mask_rows(1, t, valid_len=40)
    assert not m2[:, 40:].any()
