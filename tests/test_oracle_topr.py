"""Pins for the per-query top-keep oracle (CPU only).

Checked against things other than the oracle itself: exact integer dot
products, a hand-made case where the fp32 addition order decides the score,
the rounding-error bound of recursive summation, a brute-force statement of
the rank rule (ties to the lower index), dense attention through torch's
scaled_dot_product_attention when every key is kept, and the closed form of
a single kept key.
"""
import numpy as np
import pytest
import torch

from oracle import topr as OT


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def test_ranking_scores_exact_on_integer_data():
    g = np.random.default_rng(0)
    q = g.integers(-3, 4, (2, 3, 40, 64))
    k = g.integers(-3, 4, (2, 3, 40, 64))
    want = np.einsum("bhtd,bhsd->bhts", q, k)           # exact integers, far below 2^24
    got = OT.ranking_scores(_bf16(q), _bf16(k))
    assert got.dtype == np.float32
    assert np.array_equal(got.astype(np.int64), want)


def test_ranking_scores_add_in_order_of_d():
    """1 * 2^24 + 1 * 1 rounds back to 2^24 in fp32 (ties to even), so the
    in-order sum of [2^24, 1, -2^24] is 0; in the reverse order it is 1."""
    q = np.zeros((1, 1, 1, 64))
    q[..., :3] = 1.0
    k = np.zeros((1, 1, 2, 64))
    k[0, 0, 0, :3] = [2.0 ** 24, 1.0, -2.0 ** 24]
    k[0, 0, 1, :3] = [-2.0 ** 24, 1.0, 2.0 ** 24]
    s = OT.ranking_scores(_bf16(q), _bf16(k))
    assert s[0, 0, 0, 0] == 0.0
    assert s[0, 0, 0, 1] == 1.0


def test_ranking_scores_within_summation_bound():
    g = torch.Generator().manual_seed(1)
    q = torch.randn((1, 2, 64, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, 80, 128), generator=g).to(torch.bfloat16)
    got = OT.ranking_scores(q, k).astype(np.float64)
    qd, kd = q.double().numpy(), k.double().numpy()
    exact = np.einsum("bhtd,bhsd->bhts", qd, kd)          # fp64: every product exact, sum error ~1e-16
    absum = np.einsum("bhtd,bhsd->bhts", np.abs(qd), np.abs(kd))
    u = 2.0 ** -24
    gamma = 128 * u / (1 - 128 * u)
    assert np.all(np.abs(got - exact) <= gamma * absum + 1e-12)
    # and the scores are not exact in general: rounding happened
    assert np.any(got != exact)


def test_kept_keys_brute_force_rank_rule():
    g = np.random.default_rng(2)
    for trial in range(60):
        L = int(g.integers(1, 70))
        keep = int(g.integers(1, L + 1))
        s = g.integers(-4, 5, L).astype(np.float32)          # many ties
        got = OT.kept_keys(s, keep)
        want = [j for j in range(L)
                if sum(1 for i in range(L) if s[i] > s[j] or (s[i] == s[j] and i < j)) < keep]
        assert got.tolist() == want, (trial, L, keep)


def test_mask_keeps_exactly_keep_keys_per_query():
    g = torch.Generator().manual_seed(3)
    q = torch.randn((1, 2, 96, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, 96, 64), generator=g).to(torch.bfloat16)
    m = OT.topr_mask(q, k, 28)
    assert np.all(m.sum(axis=-1) == 28)


def test_duplicate_keys_tie_to_lower_index():
    g = torch.Generator().manual_seed(4)
    q = torch.randn((1, 1, 8, 64), generator=g)
    k = torch.randn((1, 1, 32, 64), generator=g) * 0.1
    k[0, 0, 5] = q[0, 0, 0] * 4.0                    # the best key of query 0, twice
    k[0, 0, 19] = q[0, 0, 0] * 4.0
    m = OT.topr_mask(q.to(torch.bfloat16), k.to(torch.bfloat16), 1)
    assert np.flatnonzero(m[0, 0, 0]).tolist() == [5]
    m2 = OT.topr_mask(q.to(torch.bfloat16), k.to(torch.bfloat16), 2)
    assert np.flatnonzero(m2[0, 0, 0]).tolist() == [5, 19]


def test_keep_all_equals_dense_attention():
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn((1, 2, 64, 64), generator=g).to(torch.bfloat16) for _ in range(3))
    scale = 64 ** -0.5
    o, lse = OT.topr_attention_forward(q, k, v, 64, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(), scale=scale)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    s = scale * (q.double() @ k.double().transpose(-1, -2))
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) < 1e-12


def test_keep_one_is_the_best_key():
    g = torch.Generator().manual_seed(6)
    q, k, v = (torch.randn((1, 1, 48, 64), generator=g).to(torch.bfloat16) for _ in range(3))
    scale = 0.125
    o, lse = OT.topr_attention_forward(q, k, v, 1, scale)
    s = OT.ranking_scores(q, k)[0, 0]
    for t in range(48):
        j = int(np.argmax(s[t]))                     # first maximum: the lower index on ties
        assert np.array_equal(o[0, 0, t], v[0, 0, j].double().numpy())
        want = scale * float((q[0, 0, t].double() * k[0, 0, j].double()).sum())
        assert abs(lse[0, 0, t] - want) < 1e-12


def test_rows_equal_full_evaluation():
    g = torch.Generator().manual_seed(7)
    q, k, v = (torch.randn((2, 2, 80, 64), generator=g).to(torch.bfloat16) for _ in range(3))
    o, lse = OT.topr_attention_forward(q, k, v, 24, 0.125)
    rows = [(0, 0, 0), (1, 1, 79), (0, 1, 33), (1, 0, 64)]
    ro, rl = OT.topr_attention_forward(q, k, v, 24, 0.125, rows=rows)
    for n, (b, h, t) in enumerate(rows):
        # the same keys; only the BLAS evaluation order of one row against a block differs
        assert np.max(np.abs(ro[n] - o[b, h, t])) < 1e-14 and abs(rl[n] - lse[b, h, t]) < 1e-14


@pytest.mark.parametrize("keep", [1, 7, 40])
def test_kept_keys_dominate_dropped_keys(keep):
    """Every kept key scores at least as high as every dropped key of the row."""
    g = torch.Generator().manual_seed(keep)
    q = torch.randn((1, 1, 40, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 1, 40, 64), generator=g).to(torch.bfloat16)
    s = OT.ranking_scores(q, k)[0, 0]
    m = OT.topr_mask(q, k, keep)[0, 0]
    for t in range(40):
        if keep < 40:
            assert s[t][m[t]].min() >= s[t][~m[t]].max()
