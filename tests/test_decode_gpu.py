"""Decode parity: bsa_decode (through the C ABI) against the float64 oracle.

One new token per sequence against a block-aligned KV cache; the oracle is
oracle.block_sparse_decode (row t of the causal forward over the cached
positions the token's pattern row selects).  Tolerances as for the forward:
bf16 max-abs 2e-2 on O and LSE; fp32 ||dO||_inf / ||O||_inf <= 1e-5 and
|dLSE| <= 1e-5 * max(1, |LSE|).
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import random_block_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _make(B, H, n_cap, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, d, generator=g).to(dtype)
    k = torch.randn(B, H, n_cap, d, generator=g).to(dtype)
    v = torch.randn(B, H, n_cap, d, generator=g).to(dtype)
    return q, k, v


def _check(o, lse, ro, rl, dtype):
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(lse[~fin] == -np.inf) and np.all(o[~fin] == 0)
    if dtype == torch.bfloat16:
        assert np.abs(o - ro).max() <= 2e-2
        assert np.abs(lse[fin] - rl[fin]).max(initial=0) <= 2e-2
    else:
        assert np.abs(o - ro).max() <= 1e-5 * max(np.abs(ro).max(), 1e-30)
        assert np.abs(lse[fin] - rl[fin]).max(initial=0) <= 1e-5 * max(1, np.abs(rl).max())


def _run(q, k, v, lengths, mask, bs, dtype, per_head=False, scale=None):
    dev = torch.device("cuda")
    if per_head:
        pats = [bsa.build_pattern(k.shape[2], bs, mask=m) for m in mask]
        rp, ci = bsa.stack_head_patterns(pats)
    else:
        rp, ci = bsa.build_pattern(k.shape[2], bs, mask=mask)
    sl = torch.tensor(lengths, dtype=torch.int32)
    o, lse = bsa.decode(q.to(dev), k.to(dev), v.to(dev), sl.to(dev), rp.to(dev), ci.to(dev), bs,
                        scale=scale, per_head=per_head)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bs,d", [(32, 64), (32, 128), (64, 64), (64, 128)])
def test_decode_loglinear_ragged_lengths(dtype, bs, d):
    n_cap = 16 * bs
    lengths = [1, bs - 1, bs, bs + 1, n_cap // 2 + 3, n_cap - 1, n_cap, 7 * bs + 13]
    B, H = len(lengths), 3
    q, k, v = _make(B, H, n_cap, d, dtype, 1)
    sets = oracle.loglinear_block_sets(n_cap, bs)
    mask = oracle.block_mask_from_sets(sets)
    o, lse = _run(q, k, v, lengths, mask, bs, dtype)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs)
    _check(o, lse, ro, rl, dtype)


@pytest.mark.parametrize("seed", range(3))
def test_decode_random_mask_and_scale(seed):
    bs, d, n_cap = 32, 64, 512
    M = n_cap // bs
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, n_cap + 1, size=6)]
    q, k, v = _make(6, 2, n_cap, d, torch.bfloat16, seed + 10)
    mask = random_block_mask(M, 0.3, seed)
    o, lse = _run(q, k, v, lengths, mask, bs, torch.bfloat16, scale=0.2)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs, scale=0.2)
    _check(o, lse, ro, rl, torch.bfloat16)


def test_decode_per_head_patterns():
    bs, d, n_cap, H = 64, 128, 1024, 4
    M = n_cap // bs
    masks = [random_block_mask(M, 0.25 + 0.15 * h, 20 + h) for h in range(H)]
    lengths = [n_cap, 300, 64, 65]
    q, k, v = _make(len(lengths), H, n_cap, d, torch.bfloat16, 5)
    o, lse = _run(q, k, v, lengths, masks, bs, torch.bfloat16, per_head=True)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, np.stack(masks), bs)
    _check(o, lse, ro, rl, torch.bfloat16)


def test_decode_dense_rows_longer_than_64_entries():
    # local+global-style pattern with dense rows: 128 entries in the last row
    bs, d, n_cap = 32, 64, 4096
    M = n_cap // bs
    mask = np.zeros((M, M), np.uint8)
    for i in range(M):
        mask[i, max(0, i - 4):i + 5] = 1
    mask[:, 0] = 1
    mask[M - 1, :] = 1
    lengths = [n_cap, n_cap - 40, 2049, 33]
    q, k, v = _make(len(lengths), 2, n_cap, d, torch.bfloat16, 7)
    o, lse = _run(q, k, v, lengths, mask, bs, torch.bfloat16)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs)
    _check(o, lse, ro, rl, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bs,d", [(32, 64), (32, 128), (64, 64), (64, 128)])
def test_decode_garbage_after_the_token_every_shape(dtype, bs, d):
    # NaN / inf in the cache after each sequence's length, with the token at
    # the first, a middle and the last key of a load unit and of a block
    n_cap = 8 * bs
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(n_cap, bs))
    lengths = [1, 2, 17, bs - 1, bs, bs + 1, 3 * bs - 1, 5 * bs + 9, n_cap - 3, n_cap]
    q, k, v = _make(len(lengths), 2, n_cap, d, dtype, 11 + bs + d)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs)
    for b, L in enumerate(lengths):
        k[b, :, L:] = float("nan") if b % 2 else float("inf")
        v[b, :, L:] = float("inf") if b % 2 else float("nan")
    o, lse = _run(q, k, v, lengths, mask, bs, dtype)
    _check(o, lse, ro, rl, dtype)


def test_decode_ignores_cache_beyond_length_and_bad_lengths():
    bs, d, n_cap = 32, 64, 256
    M = n_cap // bs
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(n_cap, bs))
    lengths = [40, 200, 1]
    q, k, v = _make(3, 2, n_cap, d, torch.bfloat16, 9)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs)
    for b, L in enumerate(lengths):  # garbage (NaN, inf) after each sequence's length
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("inf")
    o, lse = _run(q, k, v, lengths, mask, bs, torch.bfloat16)
    _check(o, lse, ro, rl, torch.bfloat16)
    # lengths outside [1, N_cap]: O = 0, LSE = -inf
    o, lse = _run(q, k, v, [0, n_cap + 1, -5], mask, bs, torch.bfloat16)
    assert torch.all(o.float() == 0) and torch.all(lse == -math.inf)


def test_decode_token_without_visible_keys():
    bs, d, n_cap = 32, 64, 128
    mask = np.eye(4, dtype=np.uint8)
    mask[2, 2] = 0
    mask[2, 3] = 1
    lengths = [70, 100]  # token 69 in block 2 (sees nothing), token 99 in block 3
    q, k, v = _make(2, 1, n_cap, d, torch.float32, 3)
    o, lse = _run(q, k, v, lengths, mask, bs, torch.float32)
    ro, rl = oracle.block_sparse_decode(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), lengths, mask, bs)
    _check(o, lse, ro, rl, torch.float32)


def test_decode_equals_causal_forward_row_worked_example():
    # full size: the worked example's cache (N = 4096, block 32, log-linear), B = 32;
    # the decode output of the last token equals row N-1 of the causal forward
    B, H, N, d, bs = 32, 8, 4096, 64, 32
    dev = torch.device("cuda")
    g = torch.Generator("cpu").manual_seed(0)
    q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    rp, ci = bsa.build_pattern(N, bs)
    rp, ci = rp.to(dev), ci.to(dev)
    of, lf = bsa.forward(q, k, v, rp, ci, bs, causal=True)
    lengths = torch.full((B,), N, dtype=torch.int32, device=dev)
    lengths[1::2] = torch.arange(1, B // 2 + 1, dtype=torch.int32, device=dev) * 251
    od, ld = bsa.decode(q[:, :, -1].contiguous(), k, v, torch.full((B,), N, dtype=torch.int32,
                                                                   device=dev), rp, ci, bs)
    torch.cuda.synchronize()
    assert (od.float() - of[:, :, -1].float()).abs().max().item() <= 2e-2
    assert (ld - lf[:, :, -1]).abs().max().item() <= 2e-2
    # ragged lengths: compare sampled sequences with the oracle
    idx = torch.arange(B, device=dev)
    qs = q[idx, :, (lengths - 1).long()].contiguous()
    od, ld = bsa.decode(qs, k, v, lengths, rp, ci, bs)
    torch.cuda.synchronize()
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    for b in (0, 1, 3, 17, 31):
        L = int(lengths[b])
        for h in (0, 5):
            ro, rl = oracle.block_sparse_decode_head(
                qs[b, h].double().cpu().numpy(), k[b, h].double().cpu().numpy(),
                v[b, h].double().cpu().numpy(), L, mask, bs)
            assert np.abs(od[b, h].double().cpu().numpy() - ro).max() <= 2e-2
            assert abs(ld[b, h].item() - rl) <= 2e-2
