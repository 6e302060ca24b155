"""Seeded synthetic inputs for block-sparse attention.

This module only *draws* inputs.  It holds none of the method's arithmetic
(no layout rule, no attention, no routing): both the HIP path and the fp64
oracle consume the tensors it returns, and neither imports the other.

The five named workloads mirror the shapes the pages talk about:

* BERT-base heads (12 heads of width 64) at 512 and 2048 tokens -- the
  primer page's 512-token example and the 2048-token figures quoted by the
  Adaptive-Sparse-Transformer and SQA pages;
* 8192 tokens, the sequence length of the BigBird page's performance table
  (section 性能分析);
* long padded documents (16384 tokens, head width 128) for the key-padding
  mask of the primer page's code sample;
* the SQA page's LLaMA-7B head shape (32 heads of width 128) with k=64 routed
  queries and a +-32 token local window (sections 2.1 and 4).

None of the pages' datasets (GLUE, IMDb, WikiText-103, PubMed, WMT14,
genomes) is available; kernel time does not depend on token content, so
Gaussian Q/K/V of the right shape stand in for them.

Draw order per workload, from one ``torch.Generator`` seeded with
``data_seed``: Q, K, V (fp32 ``randn * sigma``, then cast to bf16 with
round-to-nearest-even for bf16 workloads), then the router weight ``w``
(fp32, routed workloads), then ``valid_len`` (padded workloads,
``randint(L//2, L+1)`` -- uniform on the inclusive range [L/2, L]).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    dtype: str                      # "f32" or "bf16": the input/output element type
    data_seed: int
    block: int = 64
    window_blocks: int = 0          # odd; self +- (window_blocks-1)/2 blocks, clipped
    global_blocks: Tuple[int, ...] = ()
    random_blocks: int = 0
    layout_seed: int = 0
    sigma: float = 1.0
    padded: bool = False            # per-batch key valid length drawn after Q/K/V
    routed_k: int = 0               # >0: routed-query variant (top-k rows attend to all keys)
    band_tokens: int = 0            # routed variant: other rows see keys with |t-s| <= band
    token: bool = False             # token-granular BigBird pattern (window band_tokens, below)
    num_global: int = 0             # token pattern: linspace global tokens
    random_tokens: int = 0          # token pattern: random tokens per row
    keep_blocks: int = 0            # > 0: content-adaptive layout keeping this many key blocks per row
    keep_tokens: int = 0            # > 0: per-query top-keep layout keeping this many keys per query
    num_candidates: int = 0         # > 0: candidate-list attention with this many predicted positions
    cand_keep: int = 0              # candidate-list attention: candidates kept per query

    @property
    def routed(self) -> bool:
        return self.routed_k > 0

    @property
    def band(self) -> bool:
        """A token-band layout without routed rows (the plain forward on a band layout)."""
        return self.band_tokens > 0 and not self.routed and not self.token

    @property
    def adaptive(self) -> bool:
        return self.keep_blocks > 0

    @property
    def topr(self) -> bool:
        return self.keep_tokens > 0

    @property
    def candidates(self) -> bool:
        return self.num_candidates > 0

    @property
    def num_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)

    def with_(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller test shapes of the same recipe)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 8x8 blocks, fp32 end to end: window self+-1 (clipped), global block 0, one random block.
    "tiny-f32-L512": Workload(
        name="tiny-f32-L512", batch=1, heads=2, seq_len=512, head_dim=64, dtype="f32",
        data_seed=0, window_blocks=3, global_blocks=(0,), random_blocks=1, layout_seed=0),
    # BigBird layout at 2048 tokens: window 3, first/last block global, 3 random blocks.
    "bigbird-L2048": Workload(
        name="bigbird-L2048", batch=8, heads=12, seq_len=2048, head_dim=64, dtype="bf16",
        data_seed=1, window_blocks=3, global_blocks=(0, 31), random_blocks=3, layout_seed=1),
    # BigBird layout at 8192 tokens (128 blocks a side): the throughput workload.
    "bigbird-L8192": Workload(
        name="bigbird-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=2, window_blocks=3, global_blocks=(0, 127), random_blocks=3, layout_seed=2),
    # Sliding window of 5 blocks + global block 0, trailing keys padded per batch entry.
    "window-pad-L16384": Workload(
        name="window-pad-L16384", batch=4, heads=16, seq_len=16384, head_dim=128, dtype="bf16",
        data_seed=3, window_blocks=5, global_blocks=(0,), random_blocks=0, layout_seed=3,
        sigma=0.5, padded=True),
    # Routed queries: per head the top-64 rows by q.w attend to every key, the rest to +-32 tokens.
    # The BigBird layout on 128-token blocks at the throughput shape (64 blocks a side).
    "bigbird128-L8192": Workload(
        name="bigbird128-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=6, block=128, window_blocks=3, global_blocks=(0, 63), random_blocks=3, layout_seed=6),
    # The BigBird layout on 32-token blocks at the throughput shape (256 blocks a side):
    # stored as 64-token tiles with per-quarter masks.
    "bigbird32-L8192": Workload(
        name="bigbird32-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=7, block=32, window_blocks=3, global_blocks=(0, 255), random_blocks=3, layout_seed=7),
    # The token-granular BigBird pattern with the BigBird page's code defaults: a window of
    # 64 tokens each side, 8 linspace global tokens, 8 random tokens per row.
    "bigbird-tok-L8192": Workload(
        name="bigbird-tok-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=8, token=True, band_tokens=64, num_global=8, random_tokens=8, layout_seed=8),
    # Content-adaptive layout: every query block keeps the 30% of key blocks (the Adaptive page's
    # r = 0.3) with the highest pooled score, chosen on the device from Q and K.
    "adaptive-L8192": Workload(
        name="adaptive-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=9, keep_blocks=38),
    # Token-granular sliding window |t - s| <= 256 (the BigBird page's 64-256 token windows)
    # at the throughput shape: a band layout through the plain forward.
    "band256-L8192": Workload(
        name="band256-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=5, band_tokens=256),
    "routed-L4096": Workload(
        name="routed-L4096", batch=1, heads=32, seq_len=4096, head_dim=128, dtype="bf16",
        data_seed=4, routed_k=64, band_tokens=32),
    # Per-query top-keep attention (the Adaptive page's importance evaluation, r = 0.3): every
    # query keeps its floor(0.3 L) = 614 best keys, chosen on the device, at a BERT-base head shape.
    "topr-L2048": Workload(
        name="topr-L2048", batch=1, heads=12, seq_len=2048, head_dim=64, dtype="bf16",
        data_seed=10, keep_tokens=614),
    # Candidate-list attention (the Adaptive page's candidate generator, k = 32, and importance
    # evaluation, r = 0.3): a Conv1d of the hidden states (width C = H D = 768) predicts 32 key
    # positions per query; every head keeps the floor(32 * 0.3) = 9 best of them.
    "candidates-L8192": Workload(
        name="candidates-L8192", batch=2, heads=12, seq_len=8192, head_dim=64, dtype="bf16",
        data_seed=11, num_candidates=32, cand_keep=9),
}

THROUGHPUT_WORKLOAD = "bigbird-L8192"


def torch_dtype(wl: Workload) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def make_inputs(wl: Workload, device: Optional[str] = None) -> dict:
    """Draw the inputs of ``wl`` on the CPU (optionally moved to ``device``).

    Returns a dict with ``q, k, v`` ([B, H, L, D], contiguous, the workload's
    dtype), ``w`` ([D] fp32, routed workloads only), ``valid_len`` ([B]
    int32, padded workloads only) and, for candidate-list workloads, ``x``
    (bf16 [B, L, C]), ``w_conv`` (fp32 [3, C, k]) and ``b_conv`` (fp32 [k]).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.data_seed)
    shape = (wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    dt = torch_dtype(wl)
    out = {}
    for name in ("q", "k", "v"):
        x = torch.randn(shape, generator=g, dtype=torch.float32) * wl.sigma
        out[name] = x.to(dt).contiguous()
    if wl.routed:
        out["w"] = torch.randn((wl.head_dim,), generator=g, dtype=torch.float32)
    if wl.padded:
        out["valid_len"] = torch.randint(wl.seq_len // 2, wl.seq_len + 1, (wl.batch,),
                                         generator=g, dtype=torch.int64).to(torch.int32)
    if wl.candidates:
        # the candidate generator's input and weights (the page's are trained; these are seeded):
        # x [B, L, C] standard normal; the weights w [3, C, k] (tap-major) normal with standard
        # deviation (L / 2k) / sqrt(3C), so that each output spreads over about L / k tokens;
        # bias j = (j + 1/2) L / k, so that the k channels spread their positions over the sequence
        C, k, L = wl.heads * wl.head_dim, wl.num_candidates, wl.seq_len
        out["x"] = torch.randn((wl.batch, L, C), generator=g, dtype=torch.float32).to(torch.bfloat16)
        out["w_conv"] = torch.randn((3, C, k), generator=g, dtype=torch.float32) * ((L / (2 * k)) / (3 * C) ** 0.5)
        out["b_conv"] = (torch.arange(k, dtype=torch.float32) + 0.5) * (L / k)
    if device is not None:
        out = {k: v.to(device) for k, v in out.items()}
    return out


def make_grad_output(wl: Workload, device: Optional[str] = None) -> torch.Tensor:
    """The upstream gradient dO for a backward pass over ``wl``: [B, H, L, D]
    standard normal (fp32 ``randn``, cast like Q/K/V), from its own generator
    seeded with ``data_seed + 1000`` so that the forward inputs are unchanged."""
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.data_seed + 1000)
    shape = (wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    x = torch.randn(shape, generator=g, dtype=torch.float32).to(torch_dtype(wl)).contiguous()
    return x if device is None else x.to(device)


def make_layer_params(wl: Workload, device: Optional[str] = None) -> dict:
    """Input and parameters of the attention layer around ``wl``'s attention:
    x [B, L, C] standard normal, w_qkv [3C, C] and w_proj [C, C] normal with
    standard deviation 1/sqrt(C) (so projections keep unit scale), biases
    b_qkv [3C] and b_proj [C] normal with standard deviation 0.1; C = H * D.
    Drawn in that order, cast to the workload's dtype, from a generator seeded
    with ``data_seed + 2000``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.data_seed + 2000)
    C = wl.heads * wl.head_dim
    dt = torch_dtype(wl)
    out = {
        "x": torch.randn((wl.batch, wl.seq_len, C), generator=g, dtype=torch.float32),
        "w_qkv": torch.randn((3 * C, C), generator=g, dtype=torch.float32) / C ** 0.5,
        "w_proj": torch.randn((C, C), generator=g, dtype=torch.float32) / C ** 0.5,
        "b_qkv": torch.randn((3 * C,), generator=g, dtype=torch.float32) * 0.1,
        "b_proj": torch.randn((C,), generator=g, dtype=torch.float32) * 0.1,
    }
    out = {k: v.to(dt).contiguous() for k, v in out.items()}
    if device is not None:
        out = {k: v.to(device) for k, v in out.items()}
    return out
