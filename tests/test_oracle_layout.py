"""Pins for the oracle's layout rule (CPU only).

Each test checks the oracle against something other than itself: published
splitmix64 outputs, hand-derived block counts, the structure the BigBird page
prescribes (global rows/columns, a symmetric window), and the statistics of a
uniform draw.  The concrete random blocks beyond that are the library's own
specification (parity unpinned by the pages).
"""
import itertools
import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import layout as OL
from workloads import WORKLOADS


def _wl_layout(name):
    wl = WORKLOADS[name]
    if wl.routed or wl.band:
        return OL.make_band_layout(wl.heads, wl.seq_len, wl.block, wl.band_tokens)
    return OL.make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, wl.global_blocks,
                          wl.random_blocks, wl.layout_seed)


def test_splitmix64_known_answers():
    expected = [int(r[0], 16) for r in read_golden("splitmix64_state0.txt")]
    assert OL.splitmix64_stream(0, len(expected)) == expected
    # sm(x) is the first output from state x
    assert OL.sm(0) == expected[0]


def test_mix64_is_a_bijection_on_samples():
    # mix64 is a composition of invertible steps: distinct inputs give distinct outputs
    xs = list(range(5000)) + [(1 << 64) - 1 - i for i in range(5000)]
    assert len({OL.mix64(x) for x in xs}) == len(xs)


@pytest.mark.parametrize("name,expected", [(r[0], int(r[1])) for r in read_golden("layout_nnz.txt")])
def test_nnz_closed_forms(name, expected):
    lay = _wl_layout(name)
    assert lay.nnz_per_head() == [expected] * lay.num_heads


@pytest.mark.parametrize("name", ["tiny-f32-L512", "bigbird-L2048", "bigbird-L8192", "window-pad-L16384"])
def test_structure(name):
    wl = WORKLOADS[name]
    lay = _wl_layout(name)
    nb = lay.nb
    G = set(wl.global_blocks)
    wh = (wl.window_blocks - 1) // 2
    for h in range(lay.num_heads):
        bm = lay.block_mask(h)
        assert bm.diagonal().all(), "every query block sees its own block"
        for g in G:
            assert bm[g].all(), "global rows see every block"
            assert bm[:, g].all(), "every row sees the global blocks"
        # window U global is symmetric
        wg = np.zeros_like(bm)
        for i in range(nb):
            for j in range(nb):
                wg[i, j] = abs(i - j) <= wh or i in G or j in G
        assert (wg == wg.T).all()
        assert (bm | wg == bm).all(), "window and global blocks are always present"
        for i in range(nb):
            row = lay.rows[h][i]
            assert row == sorted(set(row)), "ascending, no duplicates"
            if i in G:
                continue
            extra = [j for j in row if not wg[i, j]]
            n_cand = nb - int(wg[i].sum())
            assert len(extra) == min(wl.random_blocks, n_cand)


def test_window_clipping_at_edges():
    lay = OL.make_layout(1, 10 * 64, 64, 5, [], 0, 0)
    assert lay.rows[0][0] == [0, 1, 2]
    assert lay.rows[0][1] == [0, 1, 2, 3]
    assert lay.rows[0][5] == [3, 4, 5, 6, 7]
    assert lay.rows[0][9] == [7, 8, 9]


def test_wide_window_is_dense_and_r_beyond_candidates_takes_all():
    nb = 6
    lay = OL.make_layout(2, nb * 64, 64, 2 * nb - 1, [], 3, 7)
    for h in range(2):
        assert lay.block_mask(h).all()
    lay = OL.make_layout(2, nb * 64, 64, 1, [], 100, 7)   # only self in window, r huge
    for h in range(2):
        assert lay.block_mask(h).all()


def test_deterministic_and_seed_sensitive():
    a = OL.make_layout(4, 64 * 64, 64, 3, [0], 3, 11).csr()
    b = OL.make_layout(4, 64 * 64, 64, 3, [0], 3, 11).csr()
    c = OL.make_layout(4, 64 * 64, 64, 3, [0], 3, 12).csr()
    assert all((x == y).all() for x, y in zip(a, b))
    assert (a[0] == c[0]).all()                       # same counts
    assert not (a[1] == c[1]).all()                   # different random blocks
    # heads differ too
    lay = OL.make_layout(2, 64 * 64, 64, 3, [0], 3, 11)
    assert lay.rows[0] != lay.rows[1]


def _chi2(counts, expected):
    return sum((c - expected) ** 2 / expected for c in counts)


def test_random_pairs_uniform_over_subsets():
    # window = self only, no globals, r = 2 of the 7 other blocks: every 2-subset of
    # the candidate list is equally likely under a uniform draw (21 categories).
    nb, H, seed = 8, 1500, 2024
    cats = {s: 0 for s in itertools.combinations(range(nb - 1), 2)}
    for h in range(H):
        for i in range(nb):
            cand = [j for j in range(nb) if j != i]
            row = OL.row_blocks(h, i, nb, 1, [], 2, seed)
            picked = tuple(sorted(cand.index(j) for j in row if j != i))
            cats[picked] += 1
    n = H * nb
    stat = _chi2(cats.values(), n / len(cats))
    # 20 degrees of freedom: P(chi2 > 45.3) = 0.001
    assert stat < 45.3, stat


def test_random_single_pick_uniform_over_candidates():
    nb, H, seed = 16, 800, 5
    counts = [0] * (nb - 3)
    for h in range(H):
        for i in range(1, nb - 1):
            cand = [j for j in range(nb) if abs(j - i) > 1]
            (j,) = [x for x in OL.row_blocks(h, i, nb, 3, [], 1, seed) if abs(x - i) > 1]
            counts[cand.index(j)] += 1
    n = sum(counts)
    stat = _chi2(counts, n / len(counts))
    # 12 degrees of freedom: P(chi2 > 32.9) = 0.001
    assert stat < 32.9, stat


def test_band_layout_rows_and_token_counts():
    lay = OL.make_band_layout(2, 64 * 64, 64, 32)
    assert lay.rows[0][0] == [0, 1]
    assert lay.rows[1][5] == [4, 5, 6]
    assert lay.rows[0][63] == [62, 63]
    L = 64 * 64
    t = np.arange(L)
    m = lay.token_mask_rows(0, t)
    expect = np.minimum(t + 32, L - 1) - np.maximum(t - 32, 0) + 1
    assert (m.sum(axis=1) == expect).all()
    assert m.sum(axis=1)[100] == 65


@pytest.mark.parametrize("seq_len,count", [(int(r[0]), int(r[1])) for r in read_golden("page_counts.txt")])
def test_dense_mask_counts_match_pages(seq_len, count):
    nb = seq_len // 64
    lay = OL.make_layout(1, seq_len, 64, 2 * nb - 1, [], 0, 0)
    m = lay.token_mask_rows(0, np.arange(seq_len))
    assert int(m.sum()) == count


def test_csr_matches_rows():
    lay = OL.make_layout(3, 16 * 64, 64, 3, [0, 15], 2, 9)
    row_ptr, col = lay.csr()
    assert row_ptr[0] == 0 and row_ptr[-1] == len(col)
    for h in range(3):
        for i in range(16):
            r = h * 16 + i
            assert list(col[row_ptr[r]:row_ptr[r + 1]]) == lay.rows[h][i]


def test_padding_mask_counts():
    lay = OL.make_layout(1, 8 * 64, 64, 3, [], 0, 0)
    m = lay.token_mask_rows(0, np.array([0, 200, 511]), valid_len=300)
    # row 0 (block 0) sees blocks 0,1 -> keys 0..127, all < 300
    assert m[0].sum() == 128
    # row 200 (block 3) sees blocks 2..4 -> keys 128..319, valid < 300 -> 172
    assert m[1].sum() == 300 - 128
    # row 511 (block 7) sees blocks 6,7 -> keys 384..511, none valid
    assert m[2].sum() == 0
    assert math.isclose(m[1].sum(), 172)
