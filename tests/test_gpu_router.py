"""GPU parity of the router (routed-query selection) against the oracle.

The selected rows are integers and must equal the oracle's bit for bit.  The
cases cover every rows-per-thread width of the selection (L up to 1024, 2048,
4096 and 8192), ragged lengths (a partial last 64-row score tile), k = 1 and
k = L, scores that tie in large groups (the lower row wins), all-equal
scores, infinite scores, and scores spread over a wide dynamic range (most
rows share the histogram's lowest bin).
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_transformer_amd as bs
from oracle import router as OR
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bs.lib()
    yield
    torch.cuda.synchronize()


def _check(q, w, k, tag):
    _say(tag, tuple(q.shape), "k", k)
    B, H, L, D = q.shape
    rr = torch.empty((B, H, k), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(q.cuda(), w.cuda(), k, rr)
    torch.cuda.synchronize()
    want = OR.topk_rows(OR.router_scores(q, w), k)
    got = rr.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{tag}: {len(bad)} routed rows differ, first at {bad[0].tolist()}"


def _normal(B, H, L, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, L, D), generator=g).to(torch.bfloat16)
    w = torch.randn((D,), generator=g)
    return q, w


@pytest.mark.parametrize("B,H,L,D,k", [
    (1, 32, 4096, 128, 64),     # the routed benchmark shape
    (2, 3, 1000, 64, 5),        # one row per thread, ragged last tile
    (1, 2, 300, 128, 300),      # k == L
    (1, 4, 8192, 128, 256),     # eight rows per thread
    (1, 4, 8192, 64, 8192),     # k == L at the longest length
    (1, 2, 5000, 128, 1200),    # eight rows per thread, ragged
    (3, 1, 1537, 64, 1),        # two rows per thread, one row in the last tile
    (1, 3, 3001, 128, 77),      # four rows per thread, ragged
])
def test_router_normal(B, H, L, D, k):
    q, w = _normal(B, H, L, D, seed=B * 1000 + L + k)
    _check(q, w, k, f"router normal B{B} H{H} L{L} D{D} k{k}")


@pytest.mark.parametrize("k", [7, 64, 256, 300])
def test_router_ties(k):
    """Entries of q in {0, 1} and w = 1: each score is a count, so many rows tie,
    across the whole row set; the lower row wins each tie."""
    B, H, L, D = 1, 3, 3000, 64
    g = torch.Generator().manual_seed(k)
    q = (torch.rand((B, H, L, D), generator=g) < 0.05).to(torch.bfloat16)
    w = torch.ones(D)
    _check(q, w, k, f"router ties k{k}")


@pytest.mark.parametrize("k", [3, 40, 4093])
def test_router_infinite_scores(k):
    """Rows holding one +inf (or -inf) entry, with w > 0, score +inf (-inf):
    they tie among themselves; k = 3 and 40 fall inside the +inf group,
    k = L - 3 inside the -inf group."""
    B, H, L, D = 1, 2, 4096, 128
    g = torch.Generator().manual_seed(100 + k)
    q = torch.randn((B, H, L, D), generator=g)
    w = torch.rand((D,), generator=g) + 0.1
    pos = torch.randperm(L, generator=g)
    q[:, :, pos[:50], 7] = float("inf")
    q[:, :, pos[50:60], 99] = float("-inf")
    _check(q.to(torch.bfloat16), w, k, f"router infinite k{k}")


@pytest.mark.parametrize("L,k", [(4096, 64), (8192, 300)])
def test_router_wide_dynamic_range(L, k):
    """Rows scaled by 2^e, e uniform in [-100, 100]: the histogram's range is
    set by a few huge scores and nearly every row falls in one bin."""
    B, H, D = 1, 2, 64
    g = torch.Generator().manual_seed(L + k)
    e = torch.randint(-100, 101, (B, H, L, 1), generator=g).double()
    q = (torch.randn((B, H, L, D), generator=g).double() * torch.pow(2.0, e)).float()
    w = torch.randn((D,), generator=g)
    _check(q.to(torch.bfloat16), w, k, f"router wide range L{L} k{k}")


def test_router_constant_scores():
    """Every score equal: the k lowest rows."""
    q = torch.full((1, 2, 2048, 128), 0.5, dtype=torch.bfloat16)
    w = torch.full((128,), 0.25)
    rr = torch.empty((1, 2, 64), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(q.cuda(), w.cuda(), 64, rr)
    torch.cuda.synchronize()
    assert np.array_equal(rr.cpu().numpy(), np.broadcast_to(np.arange(64, dtype=np.int32), (1, 2, 64)))


def test_router_workload_inputs_twice_with_shared_workspace():
    """The routed workload's own inputs, two calls sharing one workspace (the
    second on a smaller shape): the workspace carries nothing between calls."""
    wl = WORKLOADS["routed-L4096"]
    inp = make_inputs(wl)
    need = bs.bsattn_route_workspace_size(wl.batch, wl.heads, wl.seq_len, wl.routed_k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    q = inp["q"].cuda()
    w = inp["w"].cuda()
    rr = torch.empty((wl.batch, wl.heads, wl.routed_k), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(q, w, wl.routed_k, rr, workspace=ws)
    q2 = q[:, :5, :1500].contiguous()
    rr2 = torch.empty((wl.batch, 5, 40), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(q2, w, 40, rr2, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(rr.cpu().numpy(), OR.topk_rows(OR.router_scores(inp["q"], inp["w"]), wl.routed_k))
    assert np.array_equal(rr2.cpu().numpy(), OR.topk_rows(OR.router_scores(q2.cpu(), inp["w"]), 40))
