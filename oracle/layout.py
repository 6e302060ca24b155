"""Block layout of BigBird-style sparse attention, written out plainly (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix
------------------
* BigBird page ("BigBird 稀疏注意力机制解析：如何突破 Transformer 的序列长度限制"),
  section 核心实现: three patterns work together -- a few *global* positions
  that interact with every position (their rows see all keys and every row
  sees them), a *sliding window* of w neighbours on each side, and *random*
  remote links per position for connectivity.
* SQA page ("Transformer计算效率优化：SQA稀疏注意力机制详解"), sections 3.1
  and 5: the mask is stored in a block-sparse format, attention runs only on
  the non-zero blocks, and 64x64 blocks are the recommended tile.

Readings taken where the pages leave a step open
------------------------------------------------
* Granularity: blocks of ``block`` tokens (64).  Row i of head h lists the key
  blocks query block i attends to.
* Window: ``window_blocks`` is odd; half-width ``wh = (window_blocks-1)//2``.
  W(i) = {j : |i-j| <= wh, 0 <= j < nb}, clipped at the edges (no wrap, no
  shifting inward).  The page's ``triu(w).tril(-w)`` band expression is empty
  as printed; the prose (w neighbours before and after) is what is followed.
* Global: a global block's row is every block; every other row contains all
  global blocks.
* Random: ``r`` distinct blocks per row drawn from the complement of
  W(i) U G, in ascending order of candidates, by a partial Fisher-Yates
  shuffle driven by splitmix64 (a counter-based hash, so CPU and GPU agree).
  Per-row stream seed: s = sm(sm(sm(seed) ^ h) ^ i) with sm(x) the first
  splitmix64 output from state x.  Draw j (0-based) uses u_j, the (j+1)-th
  splitmix64 output from state s, and swaps candidate j with candidate
  j + (u_j mod (n-j)).  If r exceeds the n candidates, all n are taken.
  Global rows draw nothing.  The layout is per head and shared by the batch.
* Rows are sorted ascending and contain no duplicates (block-CSR).

splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the output mix is Stafford's "Mix13"): the state
advances by the golden-ratio increment 0x9E3779B97F4A7C15 and each output is
mix64(state) -- two xor-shift-multiply rounds and a final xor-shift.  All
arithmetic is modulo 2**64.

Routed-query variant (SQA page, section 2.1): rows of the router's top-k
queries see every key; every other query sees only keys within a local
window, read here as the token band |t - s| <= band (inclusive).  At block
granularity that band touches blocks i-1, i, i+1 for band <= block.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def mix64(z: int) -> int:
    """splitmix64's output function (Stafford Mix13), modulo 2**64."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def splitmix64_stream(state: int, count: int) -> List[int]:
    """The first ``count`` outputs of a splitmix64 generator whose state is ``state``."""
    out = []
    for _ in range(count):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        out.append(mix64(state))
    return out


def sm(x: int) -> int:
    """First splitmix64 output from state x."""
    return splitmix64_stream(x, 1)[0]


def row_stream_seed(seed: int, head: int, qblock: int) -> int:
    """Per-row stream state s = sm(sm(sm(seed) ^ head) ^ qblock)."""
    return sm(sm(sm(seed) ^ head) ^ qblock)


def window_blocks_of(i: int, nb: int, window_blocks: int) -> List[int]:
    wh = (window_blocks - 1) // 2
    return [j for j in range(nb) if abs(i - j) <= wh]


def random_blocks_of(seed: int, head: int, i: int, candidates: List[int], r: int) -> List[int]:
    """Partial Fisher-Yates over the ascending candidate list; returns the chosen blocks."""
    c = list(candidates)
    n = len(c)
    take = min(r, n)
    us = splitmix64_stream(row_stream_seed(seed, head, i), take)
    for j in range(take):
        t = j + us[j] % (n - j)
        c[j], c[t] = c[t], c[j]
    return c[:take]


def row_blocks(head: int, i: int, nb: int, window_blocks: int, global_blocks: Sequence[int],
               random_blocks: int, seed: int) -> List[int]:
    """Ascending key blocks of query block i in head ``head``."""
    g = sorted(set(global_blocks))
    if i in g:
        return list(range(nb))
    w = window_blocks_of(i, nb, window_blocks)
    taken = set(w) | set(g)
    candidates = [j for j in range(nb) if j not in taken]
    rnd = random_blocks_of(seed, head, i, candidates, random_blocks)
    return sorted(taken | set(rnd))


class Layout:
    """Per-head block rows plus the parameters that produced them."""

    def __init__(self, num_heads: int, seq_len: int, block: int, rows: List[List[List[int]]],
                 band_tokens: Optional[int] = None):
        self.num_heads = num_heads
        self.seq_len = seq_len
        self.block = block
        self.nb = seq_len // block
        self.rows = rows                    # rows[h][i] -> ascending list of key blocks
        self.band_tokens = band_tokens      # token band of the routed variant, else None

    def csr(self):
        """Block-CSR over all heads: row_ptr [H*nb+1], col_idx [nnz] (int32)."""
        row_ptr = [0]
        col = []
        for h in range(self.num_heads):
            for i in range(self.nb):
                col.extend(self.rows[h][i])
                row_ptr.append(len(col))
        return np.asarray(row_ptr, dtype=np.int32), np.asarray(col, dtype=np.int32)

    def nnz_per_head(self) -> List[int]:
        return [sum(len(r) for r in self.rows[h]) for h in range(self.num_heads)]

    def block_mask(self, head: int) -> np.ndarray:
        """[nb, nb] bool: True where query block i attends key block j."""
        m = np.zeros((self.nb, self.nb), dtype=bool)
        for i, row in enumerate(self.rows[head]):
            m[i, row] = True
        return m

    def token_mask_rows(self, head: int, t_rows: np.ndarray, valid_len: Optional[int] = None) -> np.ndarray:
        """[len(t_rows), L] bool token mask for the given query positions.

        Entry (t, s) is 1 iff block(s) is in the row of block(t), the key is
        not padding (s < valid_len), and for the band variant |t - s| <= band.
        """
        t_rows = np.asarray(t_rows, dtype=np.int64)
        bm = self.block_mask(head)
        s = np.arange(self.seq_len)
        m = bm[t_rows // self.block][:, s // self.block]
        if self.band_tokens is not None:
            m &= np.abs(t_rows[:, None] - s[None, :]) <= self.band_tokens
        if valid_len is not None:
            m &= (s < valid_len)[None, :]
        return m


def make_layout(num_heads: int, seq_len: int, block: int, window_blocks: int,
                global_blocks: Sequence[int], random_blocks: int, seed: int) -> Layout:
    if seq_len % block != 0:
        raise ValueError("seq_len must be a multiple of block")
    if window_blocks < 1 or window_blocks % 2 == 0:
        raise ValueError("window_blocks must be odd and >= 1")
    nb = seq_len // block
    if any(g < 0 or g >= nb for g in global_blocks):
        raise ValueError("global block out of range")
    rows = [[row_blocks(h, i, nb, window_blocks, global_blocks, random_blocks, seed)
             for i in range(nb)] for h in range(num_heads)]
    return Layout(num_heads, seq_len, block, rows)


def make_band_layout(num_heads: int, seq_len: int, block: int, band_tokens: int) -> Layout:
    """Blocks touched by the token band |t - s| <= band around each query block."""
    if seq_len % block != 0:
        raise ValueError("seq_len must be a multiple of block")
    nb = seq_len // block
    rows_one = []
    for i in range(nb):
        lo_tok = max(0, i * block - band_tokens)
        hi_tok = min(seq_len - 1, i * block + block - 1 + band_tokens)
        rows_one.append(list(range(lo_tok // block, hi_tok // block + 1)))
    rows = [[list(r) for r in rows_one] for _ in range(num_heads)]
    return Layout(num_heads, seq_len, block, rows, band_tokens=band_tokens)


# ---------------------------------------------------------------------------
# Token-granular BigBird pattern
# ---------------------------------------------------------------------------
# BigBird page, section 核心实现: the code example picks its global tokens
# uniformly with linspace(0, L-1, num_global) truncated to integers, every
# token attends w neighbours on each side (typical w = 64) and r random
# remote tokens (typical r = 8); the pitfalls section puts global tokens at
# 5-10% of L.  Readings:
# * global tokens G = {floor(i (L-1) / (n-1)) : 0 <= i < n} in exact integer
#   arithmetic (n = 1: {0}; n = 0: none).  The page's float32 linspace gives
#   the same integers except where rounding moves a value across an integer.
# * the pattern is the block rule above on 1-token blocks: window of 2w+1
#   tokens (|t - s| <= w), global blocks G, r random tokens per non-global row
#   drawn by the same splitmix64 partial Fisher-Yates from the tokens outside
#   the window and G, with the row stream seeded by the token index.


def linspace_tokens(seq_len: int, n: int) -> List[int]:
    """Global token positions: floor(i (L-1) / (n-1)), exact integers, ascending."""
    if n <= 0:
        return []
    if n == 1:
        return [0]
    return [(i * (seq_len - 1)) // (n - 1) for i in range(n)]


class TokenLayout:
    """Token-granular pattern, rows evaluated on demand (the block rule with block = 1).

    Row t of head h is ``row_blocks(h, t, L, 2w+1, G, r, seed)``: every token for a
    global t, else the window, the global tokens and the random tokens, ascending.
    """

    def __init__(self, num_heads: int, seq_len: int, band_tokens: int, global_tokens: Sequence[int],
                 random_tokens: int, seed: int):
        self.num_heads = num_heads
        self.seq_len = seq_len
        self.block = 1
        self.band_tokens = band_tokens
        self.global_tokens = sorted(set(int(g) for g in global_tokens))
        self.random_tokens = random_tokens
        self.seed = seed
        self._cache = {}

    def row(self, head: int, t: int) -> List[int]:
        key = (head, int(t))
        if key not in self._cache:
            self._cache[key] = row_blocks(head, int(t), self.seq_len, 2 * self.band_tokens + 1,
                                          self.global_tokens, self.random_tokens, self.seed)
        return self._cache[key]

    def random_links(self, head: int, t: int) -> List[int]:
        """The random tokens of row t (ascending; empty for a global row)."""
        if int(t) in self.global_tokens:
            return []
        g = set(self.global_tokens)
        w = self.band_tokens
        return [s for s in self.row(head, t) if abs(s - int(t)) > w and s not in g]

    def token_mask_rows(self, head: int, t_rows: np.ndarray, valid_len: Optional[int] = None) -> np.ndarray:
        """[len(t_rows), L] bool: entry (t, s) is 1 iff s is in row t (and s < valid_len)."""
        t_rows = np.asarray(t_rows, dtype=np.int64)
        m = np.zeros((len(t_rows), self.seq_len), dtype=bool)
        for n, t in enumerate(t_rows):
            m[n, self.row(head, int(t))] = True
        if valid_len is not None:
            m &= (np.arange(self.seq_len) < valid_len)[None, :]
        return m


def make_token_layout(num_heads: int, seq_len: int, band_tokens: int, num_global: int,
                      random_tokens: int, seed: int) -> TokenLayout:
    if band_tokens < 0 or band_tokens >= seq_len:
        raise ValueError("band_tokens must be in [0, seq_len)")
    if num_global < 0 or num_global > seq_len:
        raise ValueError("num_global must be in [0, seq_len]")
    if random_tokens < 0:
        raise ValueError("random_tokens must be >= 0")
    return TokenLayout(num_heads, seq_len, band_tokens, linspace_tokens(seq_len, num_global),
                       random_tokens, seed)
