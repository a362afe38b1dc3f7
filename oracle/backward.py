"""Oracle: gradients of block-sparse attention in float64 (test infrastructure only).

The backward pass is the next step after the forward that the log-linear page
points to ([P1] section 5.3 speaks of the backward of the same sparse
attention; its gradient "compensation" heuristic is not part of this).  What
is computed is the plain gradient of the forward in oracle.attention: with
P the softmax of scale * Q K^T over the visible keys of each query row (the
selected blocks, and with causal masking the keys up to the query), O = P V,
and an upstream gradient dO:

    dV = P^T dO
    dP = dO V^T
    D_r = sum_j P_rj dP_rj            (= dO_r . O_r)
    dS = P * (dP - D)                 (elementwise, D broadcast over keys)
    dQ = scale * dS K
    dK = scale * dS^T Q

written out one query block of rows at a time (no N x N matrix is held).

Pins (tests/test_oracle.py): central finite differences of the scalar
sum(G * O) with respect to every entry of Q, K and V on small inputs; torch
autograd through scaled_dot_product_attention in float64 for an all-ones
mask, a causal all-ones mask and a token-expanded block mask; D against
dO . O.
"""

from __future__ import annotations

import math

import numpy as np


def block_sparse_attention_backward_head(q, k, v, do, block_mask, block_size: int,
                                         scale: float | None = None, causal: bool = False):
    """One (batch, head): q, k, v, do are [N, d].  Returns (dQ, dK, dV, D), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    if N % block_size != 0:
        raise ValueError("N must be a multiple of block_size")
    M = N // block_size
    block_mask = np.asarray(block_mask)
    if block_mask.shape != (M, M):
        raise ValueError("block mask shape does not match N / block_size")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    dvec = np.zeros(N)
    key_pos = np.arange(N)
    for qb in range(M):
        rows = slice(qb * block_size, (qb + 1) * block_size)
        visible = np.broadcast_to(np.repeat(block_mask[qb] != 0, block_size),
                                  (block_size, N)).copy()
        if causal:
            visible &= key_pos[None, :] <= np.arange(qb * block_size,
                                                     (qb + 1) * block_size)[:, None]
        scores = (q[rows] @ k.T) * scale
        scores[~visible] = -np.inf
        has = visible.any(axis=1)
        m = np.where(has, scores.max(axis=1), 0.0)[:, None]
        p = np.exp(scores - m)
        l = p.sum(axis=1, keepdims=True)
        p = p / np.where(l > 0, l, 1.0)  # a row with no visible key has P = 0
        dv += p.T @ do[rows]
        dp = do[rows] @ v.T
        dvec[rows] = (p * dp).sum(axis=1)
        ds = p * (dp - dvec[rows][:, None])
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return dq, dk, dv, dvec


def block_sparse_attention_backward(q, k, v, do, block_mask, block_size: int,
                                    scale: float | None = None, causal: bool = False, heads=None):
    """Batched wrapper over [B, H, N, d]; ``block_mask`` is [M, M] or [H, M, M].
    Returns (dQ, dK, dV [B, H, N, d], D [B, H, N]); pairs not in ``heads`` are NaN."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    block_mask = np.asarray(block_mask)
    per_head = block_mask.ndim == 3
    out = [np.full((B, H, N, d), np.nan) for _ in range(3)]
    dvec = np.full((B, H, N), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        g = block_sparse_attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                 block_mask[h] if per_head else block_mask,
                                                 block_size, scale, causal)
        for t, x in zip(out, g[:3]):
            t[b, h] = x
        dvec[b, h] = g[3]
    return out[0], out[1], out[2], dvec
