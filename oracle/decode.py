"""Oracle: single-token decode against a block-aligned KV cache, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  Decoding is where the pages put their headline numbers
(the log-linear page, section 1: KV-cache size and latency at length 4096);
none of them spells the decode step out, so this is the plainest reading of
the forward's definition for one new token.  The KV cache of sequence b holds
L_b tokens; the new token is the last of them, at position t = L_b - 1, in
query block i = t // bs.  It attends, as row t of the causal forward does, to
the cached positions p <= t whose block p // bs the pattern row S(i) selects
(the log-linear page, section 3.3: the softmax runs over the connected blocks
only; the Ascend CANN article, "the O(N^2) bottleneck of long sequences", for
softmax(q K^T / sqrt(d)) V):

    s_p = scale * q . K_p          for the visible positions p
    m = max_p s_p,  P_p = exp(s_p - m),  l = sum_p P_p
    O = (sum_p P_p V_p) / l,  LSE = m + ln(l)

A token that sees no position (its own block not selected and no earlier
block either) gets O = 0 and LSE = -inf, as the causal forward gives such a
row.

Pins (tests/test_oracle.py): torch's scaled_dot_product_attention in float64
on the cache prefix with the token-expanded boolean mask; LSE against
scipy.special.logsumexp of the visible scores; q = 0 (uniform weights: O is
the mean of the visible V rows and LSE = ln(count)); a textbook loop over
the positions for tiny sizes.
"""

from __future__ import annotations

import math

import numpy as np


def block_sparse_decode_head(q, k_cache, v_cache, length: int, block_mask, block_size: int,
                             scale: float | None = None):
    """One (batch, head): q [d], k_cache / v_cache [N_cap, d], ``length`` = L.

    ``block_mask`` is the [M, M] pattern of the cache capacity
    (M = N_cap / block_size).  Returns (O [d] float64, LSE float).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    v = np.asarray(v_cache, dtype=np.float64)
    n_cap, d = k.shape
    if n_cap % block_size != 0:
        raise ValueError("cache capacity must be a multiple of block_size")
    if not 1 <= length <= n_cap:
        raise ValueError("length must lie in [1, cache capacity]")
    M = n_cap // block_size
    block_mask = np.asarray(block_mask)
    if block_mask.shape != (M, M):
        raise ValueError("block mask shape does not match the cache capacity")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    t = length - 1
    i = t // block_size
    positions = np.arange(length)
    visible = block_mask[i][positions // block_size] != 0
    if not visible.any():
        return np.zeros(d), -math.inf
    kv = k[:length][visible]
    vv = v[:length][visible]
    s = (kv @ q) * scale
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ vv) / l, m + math.log(l)


def block_sparse_decode(q, k_cache, v_cache, lengths, block_mask, block_size: int,
                        scale: float | None = None):
    """q [B, H, d], caches [B, H, N_cap, d], lengths [B] (ints), block_mask [M, M]
    or [H, M, M].  Returns (O [B, H, d], LSE [B, H]) in float64."""
    q = np.asarray(q)
    B, H, d = q.shape
    block_mask = np.asarray(block_mask)
    out = np.zeros((B, H, d))
    lse = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            mask_h = block_mask[h] if block_mask.ndim == 3 else block_mask
            out[b, h], lse[b, h] = block_sparse_decode_head(
                q[b, h], k_cache[b, h], v_cache[b, h], int(lengths[b]), mask_h, block_size, scale)
    return out, lse
