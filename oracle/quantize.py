"""Oracle: int8 K/V with one scale per block, and decode on such a cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The log-linear page (section 6.3, edge deployment) stores the KV cache in
int8 and computes attention in 16-bit floating point, with one quantisation
scale per block (it gives the log-stride blocks coarser scales than the local
ones: a choice of scale values, which per-block scales leave to the caller).
The page fixes no quantiser.  The plainest one is taken: symmetric, one scale
per (batch, head, block of block_size positions) over all d features:

    amax  = max |x| over the block                     (float32, exact)
    scale = amax / 127                                  (float32 division)
    code  = clip(rint(x / scale), -127, 127)            (float32 division,
                                                          ties to even)
    code  = 0 and scale = 0 for an all-zero block

Codes are integers decided in floating point, so the float32 steps above are
the definition (the library takes the same decisions in the same precision).
Dequantisation is code * scale; the attention oracles run on the dequantised
values in float64.

Pins (tests/test_oracle.py): a closed form (values k / 64 with amax 127 / 64
have scale exactly 1/64 and codes exactly k); the element of largest
magnitude maps to +-127; every code within [-127, 127] and every value within
half a scale step of its dequantisation; an all-zero block; and decode on a
dequantised cache against masked SDPA on the same values.
"""

from __future__ import annotations

import numpy as np

from .decode import block_sparse_decode


def quantize_blocks(x, block_size: int):
    """x [..., N, d] (any float dtype; taken as float32) -> (codes int8 [..., N, d],
    scales float32 [..., N / block_size])."""
    x = np.asarray(x, dtype=np.float32)
    *lead, n, d = x.shape
    if n % block_size != 0:
        raise ValueError("N must be a multiple of block_size")
    m = n // block_size
    xb = x.reshape(*lead, m, block_size, d)
    amax = np.abs(xb).max(axis=(-2, -1))                       # float32, exact
    scale = (amax / np.float32(127.0)).astype(np.float32)      # one float32 division
    codes = np.zeros_like(xb, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        s = np.where(nz, scale, np.float32(1.0))[..., None, None].astype(np.float32)
        q = np.rint((xb / s).astype(np.float32))               # float32 division, ties to even
        q = np.clip(q, -127, 127)
        codes = np.where(nz[..., None, None], q, 0).astype(np.int8)
    return codes.reshape(*lead, n, d), scale


def dequantize_blocks(codes, scales, block_size: int):
    """codes int8 [..., N, d], scales [..., N / block_size] -> float64 [..., N, d]."""
    codes = np.asarray(codes, dtype=np.float64)
    scales = np.asarray(scales, dtype=np.float64)
    per_row = np.repeat(scales, block_size, axis=-1)
    return codes * per_row[..., None]


def block_sparse_decode_int8(q, k_codes, k_scales, v_codes, v_scales, lengths, block_mask,
                             block_size: int, scale: float | None = None):
    """Decode (oracle.decode) on the dequantised caches."""
    k = dequantize_blocks(k_codes, k_scales, block_size)
    v = dequantize_blocks(v_codes, v_scales, block_size)
    return block_sparse_decode(q, k, v, lengths, block_mask, block_size, scale)
