"""fp64 CPU oracle for block-sparse attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously correct statement of what the HIP path
computes.  It is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it.  The
product path (``block_sparse_transformer_amd``) never imports it and has no
CPU fallback; the oracle shares no code, table or constant generator with the
HIP sources.

Modules
-------
``layout``    the block layout rule (sliding window + global + hash-random
              blocks) written out with plain Python lists, expanded to a
              0/1 token mask; the token-granular pattern (linspace global
              tokens, a token window, random tokens) as that rule on
              1-token blocks.
``attention`` dense masked softmax attention in fp64 from that mask.
``router``    the routed-query selection: exact fp64 score q.w and top-k.
``attention_grad``  the gradients (dQ, dK, dV) of the masked attention for
              an upstream dO: the softmax Jacobian written out in fp64.
``layer``     the attention layer around it: qkv projection, head split,
              attention, head concatenation, output projection.
``adaptive``  the content-adaptive block layout (top blocks per query block
              by pooled fp64 scores) and its attention.
``topr``      per-query top-keep attention: each query keeps its ``keep``
              best keys by an in-order fp32 score, ties to the lower index.
``candidates`` candidate-list attention: a convolution of the hidden states
              predicts key positions per query (fp64, fixed order), the best
              of them by the same fp32 score are kept and attended to.

Parity pins (see ``tests/test_oracle_*.py``): every function is checked
against something other than itself -- published splitmix64 outputs, closed
form layout counts, library routines (``scaled_dot_product_attention`` and
torch autograd in fp64), brute-force loops, central finite differences,
exact rational arithmetic and closed forms and invariants of the softmax.
Parity unpinned: the concrete choice of random blocks beyond the
hash stream itself (the composition of the per-row seed and the shuffle are
this library's own specification; any uniform draw satisfies the pages).
"""
from . import layout, attention, attention_grad, layer, router, adaptive, topr, candidates  # noqa: F401
