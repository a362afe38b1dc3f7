"""Oracle: block-sparse attention forward in float64 (test infrastructure only).

What is computed ([P3] "the O(N^2) bottleneck of long sequences": attention is
softmax(Q K^T / sqrt(d)) V; [P1] section 3.3: for each query position the
softmax runs only over the K blocks that query block is connected to, and the
denominator sums exp(score) over those positions only):

    for each (batch, head) and each query block qb:
        S   = Q[qb rows] @ K^T * scale                    (bs x N)
        S[:, token not in a selected block of qb] = -inf
        m   = max_j S,  P = exp(S - m),  l = sum_j P
        O   = (P @ V) / l,   LSE = m + ln(l)

This is dense masked attention with the block mask expanded to tokens: the
plain definition, with no blocking beyond one query block of rows at a time
(so N x N scores are never held).  Inputs are upcast exactly to float64 from
whatever precision the caller rounded them to.

LSE is the natural-log log-sum-exp of the *scaled* scores over the selected
positions (the pages do not define it; this is the plainest reading).

Causal variant (a next step the pages point to for decoding, not one they
define): query position r also drops every key position after r; a row left
with no key gets O = 0 and LSE = -inf.  Per-head patterns: ``block_mask`` may
be [H, M, M], one mask per head.

Pins (tests/test_oracle.py): causal all-ones against torch's causal
scaled_dot_product_attention and a causal textbook loop; causal Q = 0
(uniform weights over the visible keys, LSE = ln(count)); an all-ones mask against torch's
scaled_dot_product_attention in float64 and against a textbook loop; a general
block mask against scaled_dot_product_attention with the token-expanded
boolean mask; per-block dense attention for a diagonal mask; Q = 0 (uniform
weights: O = mean of selected V rows, LSE = ln(bs * |S|)); V constant; LSE
against scipy.special.logsumexp; convex-combination invariants (weights zero
outside the selection, row sums 1 to 1e-12 -- [P1] section 3.3 asks for
0.999..1.001).
"""

from __future__ import annotations

import math

import numpy as np


def block_sparse_attention_head(q, k, v, block_mask, block_size: int, scale: float | None = None,
                                query_blocks=None, return_weights: bool = False,
                                causal: bool = False):
    """One (batch, head): q, k, v are [N, d] arrays of any float dtype.

    ``block_mask`` is [M, M] (nonzero = selected), M = N / block_size.
    ``query_blocks`` restricts the work to those query blocks (default: all);
    rows of O/LSE outside them are left as NaN.  ``causal`` also hides keys
    after each query position.
    Returns (O [N, d] float64, LSE [N] float64[, W dict qb -> [bs, N] weights]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    if N % block_size != 0:
        raise ValueError("N must be a multiple of block_size")
    M = N // block_size
    block_mask = np.asarray(block_mask)
    if block_mask.shape != (M, M):
        raise ValueError("block mask shape does not match N / block_size")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if query_blocks is None:
        query_blocks = range(M)

    out = np.full((N, d), np.nan, dtype=np.float64)
    lse = np.full((N,), np.nan, dtype=np.float64)
    weights = {}
    key_pos = np.arange(N)
    for qb in query_blocks:
        rows = slice(qb * block_size, (qb + 1) * block_size)
        token_selected = np.repeat(block_mask[qb] != 0, block_size)  # [N]
        if not token_selected.any():
            raise ValueError(f"query block {qb} selects no K block")
        visible = np.broadcast_to(token_selected, (block_size, N)).copy()  # [bs, N]
        if causal:
            query_pos = np.arange(qb * block_size, (qb + 1) * block_size)[:, None]
            visible &= key_pos[None, :] <= query_pos
        scores = (q[rows] @ k.T) * scale  # [bs, N]
        scores[~visible] = -np.inf
        m = scores.max(axis=1, keepdims=True)
        empty = ~visible.any(axis=1)
        m[empty] = 0.0  # a row with no visible key: O = 0, LSE = -inf
        p = np.exp(scores - m)  # exp(-inf) = 0 outside the selection
        l = p.sum(axis=1, keepdims=True)
        safe_l = np.where(l > 0, l, 1.0)
        out[rows] = (p @ v) / safe_l
        with np.errstate(divide="ignore"):
            lse[rows] = np.where(l[:, 0] > 0, (m + np.log(safe_l))[:, 0], -np.inf)
        if return_weights:
            weights[qb] = p / safe_l
    if return_weights:
        return out, lse, weights
    return out, lse


def block_sparse_attention(q, k, v, block_mask, block_size: int, scale: float | None = None,
                           heads=None, query_blocks=None, causal: bool = False):
    """Batched wrapper: q, k, v are [B, H, N, d].

    ``block_mask`` is [M, M] (one pattern for all heads) or [H, M, M] (one per
    head).  ``heads`` is an iterable of (b, h) pairs to evaluate (default:
    all).  Returns (O [B, H, N, d] float64, LSE [B, H, N] float64); entries
    that were not evaluated are NaN.
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    block_mask = np.asarray(block_mask)
    per_head = block_mask.ndim == 3
    if per_head and block_mask.shape[0] != H:
        raise ValueError("a per-head block mask needs one [M, M] mask per head")
    out = np.full((B, H, N, d), np.nan, dtype=np.float64)
    lse = np.full((B, H, N), np.nan, dtype=np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        mask_h = block_mask[h] if per_head else block_mask
        o_bh, lse_bh = block_sparse_attention_head(q[b, h], k[b, h], v[b, h], mask_h,
                                                   block_size, scale, query_blocks,
                                                   causal=causal)
        out[b, h] = o_bh
        lse[b, h] = lse_bh
    return out, lse
