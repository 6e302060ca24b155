"""Pins for the oracle's router (CPU only).

The score is checked with exact rational arithmetic (products are exact; the
sum is within the classical bound of a recursive fp64 summation) and with a
hand-computed case where the left-to-right order decides the result.  The
top-k is checked against a full stable sort and hand-made ties.
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import router as OR


def test_products_exact_and_sum_within_recursive_bound():
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 2, 64, 128, generator=g).to(torch.bfloat16)
    w = torch.randn(128, generator=g)
    s = OR.router_scores(q, w)
    qd = q.double().numpy()
    wd = w.double().numpy()
    u = 2.0 ** -53
    n = 127
    gamma = n * u / (1 - n * u)
    for h in range(2):
        for t in range(0, 64, 7):
            terms = [Fraction(float(qd[0, h, t, d])) * Fraction(float(wd[d])) for d in range(128)]
            for d in range(128):
                assert Fraction(float(qd[0, h, t, d] * wd[d])) == terms[d]   # exact products
            exact = sum(terms)
            bound = gamma * float(sum(abs(x) for x in terms))
            assert abs(Fraction(float(s[0, h, t])) - exact) <= Fraction(bound)


def test_left_to_right_order_by_hand():
    # q = [1, 2^53, -2^53, 0...], w = 1: sequentially 1 + 2^53 rounds (ties-to-even) to 2^53,
    # then 2^53 - 2^53 = 0.  Any other grouping that adds 2^53 and -2^53 first gives 1.
    q = torch.zeros(1, 1, 1, 8, dtype=torch.bfloat16)
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 0, 1] = 2.0 ** 53
    q[0, 0, 0, 2] = -(2.0 ** 53)
    w = torch.ones(8)
    assert OR.router_scores(q, w)[0, 0, 0] == 0.0
    # and with the big terms first the same definition gives 1
    q2 = torch.zeros(1, 1, 1, 8, dtype=torch.bfloat16)
    q2[0, 0, 0, 0] = 2.0 ** 53
    q2[0, 0, 0, 1] = -(2.0 ** 53)
    q2[0, 0, 0, 2] = 1.0
    assert OR.router_scores(q2, w)[0, 0, 0] == 1.0


def test_topk_hand_ties():
    s = np.array([[[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]]])
    assert OR.topk_rows(s, 2).tolist() == [[[1, 2]]]
    assert OR.topk_rows(s, 3).tolist() == [[[1, 2, 4]]]
    assert OR.topk_rows(s, 4).tolist() == [[[1, 2, 3, 4]]]


def test_topk_matches_full_sort():
    g = np.random.default_rng(3)
    s = np.round(g.standard_normal((2, 3, 300)), 1)        # many ties
    got = OR.topk_rows(s, 17)
    for b in range(2):
        for h in range(3):
            full = sorted(range(300), key=lambda t: (-s[b, h, t], t))
            assert got[b, h].tolist() == sorted(full[:17])
