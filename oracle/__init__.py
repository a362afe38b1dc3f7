"""CPU oracle for log-linear block-sparse attention (forward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constant generators) and imports
nothing from it.

It is deliberately plain and slow:

* ``oracle.pattern`` -- the block-selection rules written out step by step
  (log-linear rule, local+global token mask and its block conversion, dilated
  window, BigBird with its counter-based draw, causal filtering) and the CSR
  encoding of a block mask, in Python integers.
* ``oracle.attention`` -- dense softmax attention in float64 with an explicit
  block mask expanded to tokens, one query block at a time.
* ``oracle.backward`` -- the plain gradients dQ, dK, dV of that forward.
* ``oracle.decode`` -- one new token against a KV cache: row t of the causal
  forward, over the cached positions its block's pattern row selects.
* ``oracle.quantize`` -- int8 K/V with one scale per block (symmetric,
  float32 decisions), dequantisation, and decode on a dequantised cache.

Sources (web pages; cited by title and section):

* [P1] "Block Sparse Attention: Log-Linear complexity sparse attention
  implementation" (czchanglian.com, news/56740): the pattern rule (section
  3.1), the precomputed per-query-block index table (section 3.2) and the
  softmax normalised over the connected blocks only (section 3.3).
* [P2] "How to implement efficient sparse attention for the 4090: from
  principle to engineering practice" (qqiyuan.cn): Bernoulli block mask
  ("core implementation logic", item 1).
* [P3] Ascend CANN SparseFlashAttention article (hwcomputing.csdn.net):
  the attention formula softmax(QK^T/sqrt(d))V ("the O(N^2) bottleneck of long
  sequences"), the local+global token mask ("sparse pattern: Local + Global")
  and its token-to-block conversion ("Block-Sparse").

Every function here is pinned by ``tests/test_oracle.py`` against something
other than itself (hand-derived worked examples, closed forms, library
routines, invariants).  Parity pins per function are listed in each module's
docstring; none is "parity unpinned".
"""

from .pattern import (
    ceil_log2,
    loglinear_block_sets,
    dilated_block_sets,
    bigbird_block_sets,
    causal_block_sets,
    splitmix64_at,
    block_mask_from_sets,
    csr_from_block_mask,
    block_mask_from_csr,
    local_global_token_mask,
    token_mask_to_block_mask,
)
from .attention import block_sparse_attention_head, block_sparse_attention
from .backward import block_sparse_attention_backward_head, block_sparse_attention_backward
from .decode import block_sparse_decode_head, block_sparse_decode
from .quantize import quantize_blocks, dequantize_blocks, block_sparse_decode_int8

__all__ = [
    "ceil_log2",
    "loglinear_block_sets",
    "dilated_block_sets",
    "bigbird_block_sets",
    "causal_block_sets",
    "splitmix64_at",
    "block_mask_from_sets",
    "csr_from_block_mask",
    "block_mask_from_csr",
    "local_global_token_mask",
    "token_mask_to_block_mask",
    "block_sparse_attention_head",
    "block_sparse_attention",
    "block_sparse_attention_backward_head",
    "block_sparse_attention_backward",
    "block_sparse_decode_head",
    "block_sparse_decode",
    "quantize_blocks",
    "dequantize_blocks",
    "block_sparse_decode_int8",
]
