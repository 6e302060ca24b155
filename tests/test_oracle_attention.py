"""Pins for the oracle's masked attention (CPU only).

Checks against a library routine (torch's scaled_dot_product_attention in
fp64 on the CPU), brute-force pure-Python loops, and closed forms of the
softmax (rows sum to one, Q = 0 gives the mean of the allowed values and
LSE = ln(count), a single allowed key returns its value, a key shift moves
LSE by the exact dot product and leaves O unchanged).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import layout as OL


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _sdpa(q, k, v, mask, scale):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    tm = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                         attn_mask=tm[None], scale=scale)
    return o[0].numpy()


def test_full_mask_equals_sdpa():
    n, D = 96, 32
    q, k, v = _rand((n, D), 1), _rand((n, D), 2), _rand((n, D), 3)
    mask = np.ones((n, n), dtype=bool)
    o, lse = OA.masked_attention(q, k, v, mask, 0.2)
    ref = _sdpa(q, k, v, mask, 0.2)
    assert np.abs(o - ref).max() < 1e-12


def test_random_mask_equals_sdpa_boolean_mask():
    n, m, D = 80, 120, 16
    q, k, v = _rand((n, D), 4), _rand((m, D), 5), _rand((m, D), 6)
    g = np.random.default_rng(7)
    mask = g.random((n, m)) < 0.2
    mask[np.arange(n), g.integers(0, m, n)] = True          # at least one key per row
    o, _ = OA.masked_attention(q, k, v, mask, 0.3)
    ref = _sdpa(q, k, v, mask, 0.3)
    assert np.abs(o - ref).max() < 1e-12


def test_layout_covering_all_blocks_is_dense_attention():
    B, H, L, D = 1, 2, 4 * 64, 16
    q, k, v = _rand((B, H, L, D), 8), _rand((B, H, L, D), 9), _rand((B, H, L, D), 10)
    lay = OL.make_layout(H, L, 64, 7, [], 0, 0)
    o, lse = OA.attention_forward(q, k, v, lay, 0.25, chunk=100)
    for h in range(H):
        ref = _sdpa(q[0, h], k[0, h], v[0, h], np.ones((L, L), dtype=bool), 0.25)
        assert np.abs(o[0, h] - ref).max() < 1e-12


def test_window_layout_matches_brute_force_loops():
    # tiny L, block 4 so the window spans several blocks; pure-Python loops with math.exp
    L, D, blk = 24, 3, 4
    q, k, v = _rand((1, 1, L, D), 11), _rand((1, 1, L, D), 12), _rand((1, 1, L, D), 13)
    lay = OL.make_layout(1, L, blk, 3, [], 0, 0)
    o, lse = OA.attention_forward(q, k, v, lay, 0.7)
    for t in range(L):
        bt = t // blk
        keys = [s for s in range(L) if abs(s // blk - bt) <= 1]
        sc = [0.7 * sum(q[0, 0, t, d] * k[0, 0, s, d] for d in range(D)) for s in keys]
        mx = max(sc)
        ws = [math.exp(x - mx) for x in sc]
        tot = sum(ws)
        for d in range(D):
            ref = sum(w * v[0, 0, s, d] for w, s in zip(ws, keys)) / tot
            assert abs(o[0, 0, t, d] - ref) < 1e-12
        assert abs(lse[0, 0, t] - (mx + math.log(tot))) < 1e-12


def test_values_all_one_gives_one():
    B, H, L, D = 1, 2, 6 * 64, 8
    q, k = _rand((B, H, L, D), 14, 3.0), _rand((B, H, L, D), 15, 3.0)
    v = np.ones((B, H, L, D))
    lay = OL.make_layout(H, L, 64, 3, [0], 1, 3)
    o, _ = OA.attention_forward(q, k, v, lay, 0.5)
    assert np.abs(o - 1.0).max() < 1e-13


def test_zero_queries_closed_form_with_padding():
    B, H, L, D = 2, 2, 8 * 64, 8
    q = np.zeros((B, H, L, D))
    k, v = _rand((B, H, L, D), 16), _rand((B, H, L, D), 17)
    lay = OL.make_layout(H, L, 64, 3, [0], 2, 4)
    valid = [L, 300]
    o, lse = OA.attention_forward(q, k, v, lay, 0.125, valid_len=valid)
    for b in range(B):
        for h in range(H):
            for t in range(0, L, 37):
                blocks = lay.rows[h][t // 64]
                keys = [s for s in range(L) if s // 64 in blocks and s < valid[b]]
                assert lse[b, h, t] == pytest.approx(math.log(len(keys)), abs=1e-14)
                assert np.abs(o[b, h, t] - v[b, h, keys].mean(axis=0)).max() < 1e-13


def test_single_allowed_key_returns_its_value():
    n, D = 10, 6
    q, k, v = _rand((n, D), 18), _rand((n, D), 19), _rand((n, D), 20)
    mask = np.zeros((n, n), dtype=bool)
    pick = (np.arange(n) * 3) % n
    mask[np.arange(n), pick] = True
    o, lse = OA.masked_attention(q, k, v, mask, 0.9)
    assert np.abs(o - v[pick]).max() < 1e-15
    for t in range(n):
        assert lse[t] == pytest.approx(0.9 * float(q[t] @ k[pick[t]]), abs=1e-14)


def test_key_shift_leaves_output_and_moves_lse():
    L, D = 5 * 64, 8
    q, k, v = _rand((1, 1, L, D), 21), _rand((1, 1, L, D), 22), _rand((1, 1, L, D), 23)
    c = _rand((D,), 24)
    lay = OL.make_layout(1, L, 64, 3, [2], 1, 5)
    o1, l1 = OA.attention_forward(q, k, v, lay, 0.3)
    o2, l2 = OA.attention_forward(q, k + c, v, lay, 0.3)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs((l2 - l1) - 0.3 * (q @ c)).max() < 1e-12


def test_rows_sum_to_one_via_linearity():
    # O is linear in V: with V = identity columns, O's rows are the attention weights
    n, D = 40, 5
    q, k = _rand((n, D), 25), _rand((n, D), 26)
    g = np.random.default_rng(27)
    mask = g.random((n, n)) < 0.3
    mask[np.arange(n), np.arange(n)] = True
    p, _ = OA.masked_attention(q, k, np.eye(n), mask, 1.0)
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-14
    assert (p[~mask] == 0).all()
    assert (p[mask] > 0).all()


def test_fully_masked_row():
    q, k, v = _rand((3, 4), 28), _rand((5, 4), 29), _rand((5, 4), 30)
    mask = np.ones((3, 5), dtype=bool)
    mask[1] = False
    o, lse = OA.masked_attention(q, k, v, mask, 1.0)
    assert (o[1] == 0).all() and np.isneginf(lse[1])
    assert np.isfinite(lse[[0, 2]]).all()


def test_rows_api_matches_full_forward():
    B, H, L, D = 2, 2, 6 * 64, 8
    q, k, v = _rand((B, H, L, D), 31), _rand((B, H, L, D), 32), _rand((B, H, L, D), 33)
    lay = OL.make_layout(H, L, 64, 3, [0, 5], 1, 6)
    valid = [L, 200]
    o, lse = OA.attention_forward(q, k, v, lay, 0.4, valid_len=valid)
    rows = [(b, h, t) for b in range(B) for h in range(H) for t in (0, 63, 64, 199, 200, L - 1)]
    ro, rl = OA.attention_rows(q, k, v, lay, 0.4, rows, valid_len=valid)
    for n, (b, h, t) in enumerate(rows):
        assert np.abs(ro[n] - o[b, h, t]).max() < 1e-14
        assert abs(rl[n] - lse[b, h, t]) < 1e-14


def test_routed_zero_queries_closed_form():
    B, H, L, D = 1, 2, 4 * 64, 4
    q = np.zeros((B, H, L, D))
    k, v = _rand((B, H, L, D), 34), _rand((B, H, L, D), 35)
    routed = np.array([[[3, 100, 255], [0, 1, 2]]])
    o, lse = OA.routed_attention_forward(q, k, v, routed, 32, 0.5)
    for h in range(H):
        for t in range(L):
            if t in routed[0, h]:
                n = L
                keys = np.arange(L)
            else:
                lo, hi = max(0, t - 32), min(L - 1, t + 32)
                n = hi - lo + 1
                keys = np.arange(lo, hi + 1)
            assert lse[0, h, t] == pytest.approx(math.log(n), abs=1e-14)
            assert np.abs(o[0, h, t] - v[0, h, keys].mean(axis=0)).max() < 1e-13


def test_band_layout_mask_equals_routed_mask_off_route():
    L = 6 * 64
    lay = OL.make_band_layout(1, L, 64, 32)
    t = np.arange(L)
    a = lay.token_mask_rows(0, t)
    b = OA.routed_token_mask_rows(t, L, [], 32)
    assert (a == b).all()
