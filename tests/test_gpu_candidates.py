"""GPU parity of candidate-list attention against the oracle.

Positions and kept keys are integer results and must equal the oracle's bit
for bit: the positions come from the fp64 fixed-order convolution on both
sides, the kept keys from the in-order fp32 ranking.  The attention output
is compared with the fp64 oracle at the bf16 tolerances (O 2e-2, LSE 1e-3).
Cases: several (C, k) shapes including a k that is not a power of two and
k = 1 and 64 (positions), forward at k = 20, 32, 48 and 64 (the two-queries-
per-wave kernel up to k = 32, the one-query kernel above), a sequence length
that does not fill the last workgroup,
rounding at the ends of the sequence and a NaN input row, positions given
directly with many repeats and values outside the sequence, keep = 1 and
keep = k, integer-valued scores (ties), D = 64 and 128, and the benchmark
shape (all positions of one batch entry, sampled rows of the forward).
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from conftest import record_parity
from oracle import candidates as OC
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bs.lib()
    yield
    torch.cuda.synchronize()


def _generator(B, L, C, k, seed, spread=None):
    """x [B, L, C] bf16, w [3, C, k] fp32 (tap-major), bias [k]: positions spread over the sequence."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, L, C), generator=g).to(torch.bfloat16)
    s = (L / (2 * k)) if spread is None else spread
    w = torch.randn((3, C, k), generator=g) * (s / (3 * C) ** 0.5)
    bias = (torch.arange(k, dtype=torch.float32) + 0.5) * (L / k)
    return x, w, bias


def _oracle_positions(x, w, bias):
    return OC.candidate_positions(x, w.permute(2, 1, 0).contiguous().numpy(), bias.numpy())


def _device_positions(x, w, bias):
    pos = bs.bsattn_candidate_positions(x.cuda(), w.cuda(), bias.cuda())
    torch.cuda.synchronize()
    return pos.cpu().numpy()


@pytest.mark.parametrize("B,L,C,k", [(2, 256, 96, 32), (1, 100, 40, 20), (1, 64, 8, 1), (1, 300, 24, 64)])
def test_positions_bit_exact(B, L, C, k):
    _say("positions", B, L, C, k)
    x, w, bias = _generator(B, L, C, k, seed=L + C + k)
    got = _device_positions(x, w, bias)
    want = _oracle_positions(x, w, bias)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} positions differ, first {bad[0].tolist()}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def test_positions_clamp_and_nan():
    """Wide spread: many outputs fall outside the sequence and clamp to 0 or L - 1;
    a NaN in one input row makes the outputs of its three neighbours 0."""
    B, L, C, k = 1, 128, 16, 32
    x, w, bias = _generator(B, L, C, k, seed=7, spread=4 * L)
    x[0, 40, 3] = float("nan")
    got = _device_positions(x, w, bias)
    want = _oracle_positions(x, w, bias)
    assert np.array_equal(got, want)
    assert (got == 0).any() and (got == L - 1).any()
    assert np.all(got[0, 39:42] == 0)


def test_positions_benchmark_shape_one_batch():
    wl = WORKLOADS["candidates-L8192"]
    inp = make_inputs(wl)
    _say("positions bench shape", wl.name)
    x = inp["x"][:1].contiguous()
    got = _device_positions(x, inp["w_conv"], inp["b_conv"])
    want = _oracle_positions(x, inp["w_conv"], inp["b_conv"])
    assert np.array_equal(got, want)


def _inputs(B, H, L, D, seed, integer=False):
    g = torch.Generator().manual_seed(seed)
    if integer:
        return tuple(torch.randint(-1, 2, (B, H, L, D), generator=g).to(torch.bfloat16) for _ in range(3))
    return tuple(torch.randn((B, H, L, D), generator=g).to(torch.bfloat16) for _ in range(3))


def _run(q, k, v, pos, keep):
    B, H, L, D = q.shape
    kept = torch.full((B, H, L, keep), -7, dtype=torch.int32, device="cuda")
    out, lse = bs.bsattn_candidate_forward(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(pos).cuda(), keep,
                                           scale=D ** -0.5, kept=kept)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), kept.cpu().numpy()


def _check_kept(q, k, pos, keep, kept, tag):
    q32, k32 = q.float().numpy(), k.float().numpy()
    B, H, L, _ = q.shape
    for b in range(B):
        for h in range(H):
            for t in range(L):
                p = pos[b, t]
                p = p[(p >= 0) & (p < L)]
                want = OC.kept_candidates(q32[b, h, t], k32[b, h], p, keep) if p.size else np.zeros(0, np.int64)
                row = np.full(keep, -1)
                row[:len(want)] = want
                assert np.array_equal(kept[b, h, t], row), f"{tag}: kept keys of {(b, h, t)} differ"


def _check_forward(q, k, v, pos, keep, out, lse, tag, rows=None):
    B, H, L, D = q.shape
    scale = D ** -0.5
    if rows is None:
        ro, rl = OC.candidate_attention_forward(q, k, v, pos, keep, scale)
        go, gl = out, lse
    else:
        ro, rl = OC.candidate_attention_forward(q, k, v, pos, keep, scale, rows=rows)
        go = np.stack([out[b, h, t] for b, h, t in rows])
        gl = np.array([lse[b, h, t] for b, h, t in rows])
    eo, el = float(np.max(np.abs(go - ro))), float(np.max(np.abs(gl - rl)))
    print(f"  {tag}: O {eo:.2e} / {TOL_O:g}  LSE {el:.2e} / {TOL_LSE:g}", file=sys.stderr, flush=True)
    record_parity(tag, "O", eo, TOL_O)
    record_parity(tag, "LSE", el, TOL_LSE)
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O {eo:.3e} LSE {el:.3e}"


@pytest.mark.parametrize("D,keep", [(64, 9), (128, 9), (64, 1), (64, 32)])
def test_forward_from_generated_positions(D, keep):
    B, H, L, k, C = 2, 2, 256, 32, 48
    tag = f"candidates D={D} keep={keep}"
    _say(tag)
    x, w, bias = _generator(B, L, C, k, seed=D + keep)
    pos = _device_positions(x, w, bias)
    q, kk, v = _inputs(B, H, L, D, seed=3 * D + keep)
    out, lse, kept = _run(q, kk, v, pos, keep)
    _check_kept(q, kk, pos, keep, kept, tag)
    _check_forward(q, kk, v, pos, keep, out, lse, tag)


@pytest.mark.parametrize("D,k,keep,L", [(64, 20, 5, 200), (64, 48, 12, 200), (128, 64, 16, 200), (64, 32, 9, 101)])
def test_forward_other_candidate_counts(D, k, keep, L):
    """k not a power of two (two queries per wave), k above 32 (one query per wave), and an odd
    sequence length, whose last wave has no second query."""
    B, H, C = 1, 2, 24
    tag = f"candidates D={D} k={k} keep={keep} L={L}"
    _say(tag)
    x, w, bias = _generator(B, L, C, k, seed=D + k + keep + L)
    pos = _device_positions(x, w, bias)
    q, kk, v = _inputs(B, H, L, D, seed=5 * k + keep)
    out, lse, kept = _run(q, kk, v, pos, keep)
    _check_kept(q, kk, pos, keep, kept, tag)
    _check_forward(q, kk, v, pos, keep, out, lse, tag)


def test_repeats_and_out_of_range_positions():
    """Positions given directly: drawn from 6 values, so most repeat, and some outside the
    sequence (ignored); one query has none in range (O = 0, LSE = -inf)."""
    B, H, L, D, k, keep = 1, 2, 64, 64, 16, 4
    g = np.random.default_rng(9)
    pos = g.choice([-3, 5, 17, 17, 40, 63, 70], size=(B, L, k)).astype(np.int32)
    pos[0, 10] = -1
    q, kk, v = _inputs(B, H, L, D, seed=21)
    out, lse, kept = _run(q, kk, v, pos, keep)
    _check_kept(q, kk, pos, keep, kept, "candidates repeats")
    assert np.all(kept[0, :, 10] == -1) and np.all(out[0, :, 10] == 0) and np.all(np.isneginf(lse[0, :, 10]))
    # the forward of every other query, against the oracle on its in-range positions
    eo = el = 0.0
    for h in range(H):
        for t in range(L):
            if t == 10:
                continue
            p = pos[0, t]
            p = p[(p >= 0) & (p < L)]
            ro, rl = OC.candidate_attention_forward(q, kk, v, np.broadcast_to(p, (1, L, p.size)).copy(), keep,
                                                    D ** -0.5, rows=[(0, h, t)])
            eo = max(eo, float(np.max(np.abs(out[0, h, t] - ro[0]))))
            el = max(el, abs(float(lse[0, h, t] - rl[0])))
    record_parity("candidates repeats", "O", eo, TOL_O)
    record_parity("candidates repeats", "LSE", el, TOL_LSE)
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


def test_integer_scores_tie_to_lower_position():
    B, H, L, D, k, keep = 1, 1, 128, 64, 32, 9
    x, w, bias = _generator(B, L, 16, k, seed=31)
    pos = _device_positions(x, w, bias)
    q, kk, v = _inputs(B, H, L, D, seed=32, integer=True)
    out, lse, kept = _run(q, kk, v, pos, keep)
    _check_kept(q, kk, pos, keep, kept, "candidates integer scores")


def test_benchmark_shape_sampled():
    wl = WORKLOADS["candidates-L8192"]
    _say("candidates bench shape", wl.name)
    inp = make_inputs(wl)
    pos = _device_positions(inp["x"], inp["w_conv"], inp["b_conv"])
    q, kk, v = inp["q"], inp["k"], inp["v"]
    out, lse, kept = _run(q, kk, v, pos, wl.cand_keep)
    g = np.random.default_rng(15)
    rows = [(int(g.integers(wl.batch)), int(g.integers(wl.heads)), int(t))
            for t in list(g.integers(0, wl.seq_len, 40)) + [0, 1, wl.seq_len - 1]]
    q32, k32 = q.float().numpy(), kk.float().numpy()
    for b, h, t in rows:
        want = OC.kept_candidates(q32[b, h, t], k32[b, h], pos[b, t], wl.cand_keep)
        row = np.full(wl.cand_keep, -1)
        row[:len(want)] = want
        assert np.array_equal(kept[b, h, t], row), (b, h, t)
    _check_forward(q, kk, v, pos, wl.cand_keep, out, lse, "candidates-L8192 sampled rows", rows=rows)
