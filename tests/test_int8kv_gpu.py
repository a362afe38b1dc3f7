"""int8 K/V with per-block scales: the quantiser (bit-exact against the
oracle's float32 decisions) and decode on an int8 cache (against the float64
oracle on the dequantised cache).  Codes and scales fed to the decode come
from the oracle's quantiser, never from the GPU's."""

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


def _randn(shape, dtype, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bs,d", [(32, 64), (32, 128), (64, 64), (64, 128)])
def test_quantize_bit_exact(dtype, bs, d):
    B, H, N = 2, 3, 8 * bs
    x = _randn((B, H, N, d), dtype, bs + d)
    x[0, 1, bs:2 * bs] = 0          # an all-zero block
    x[1, 2, :bs] *= 1e-3            # a small-scale block
    x[1, 0, 3 * bs:4 * bs] *= 50.0  # a large-scale block
    codes, scales = bsa.quantize_kv(x.cuda(), bs)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_blocks(x.float().numpy(), bs)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_full_size_cache_bit_exact():
    # the worked example's cache: B=32, H=8, N=4096, d=64, block 32
    B, H, N, d, bs = 32, 8, 4096, 64, 32
    x = _randn((B, H, N, d), torch.bfloat16, 0)
    codes, scales = bsa.quantize_kv(x.cuda(), bs)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (31, 7), (13, 4)):
        rc, rs = oracle.quantize_blocks(x[b, h].float().numpy(), bs)
        assert np.array_equal(scales[b, h].cpu().numpy(), rs)
        assert np.array_equal(codes[b, h].cpu().numpy(), rc)


def _decode_case(B, H, n_cap, d, bs, dtype, lengths, mask, seed, per_head=False, scale=None):
    q = _randn((B, H, d), dtype, seed)
    k = _randn((B, H, n_cap, d), torch.float32, seed + 1)
    v = _randn((B, H, n_cap, d), torch.float32, seed + 2)
    kc, ks = oracle.quantize_blocks(k.numpy(), bs)
    vc, vs = oracle.quantize_blocks(v.numpy(), bs)
    dev = torch.device("cuda")
    if per_head:
        rp, ci = bsa.stack_head_patterns([bsa.build_pattern(n_cap, bs, mask=m) for m in mask])
    else:
        rp, ci = bsa.build_pattern(n_cap, bs, mask=mask)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, lse = bsa.decode_int8kv(q.to(dev), t(kc), t(ks), t(vc), t(vs),
                               torch.tensor(lengths, dtype=torch.int32, device=dev),
                               rp.to(dev), ci.to(dev), bs, scale=scale, per_head=per_head)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_decode_int8(q.double().numpy(), kc, ks, vc, vs, lengths,
                                             np.stack(mask) if per_head else mask, bs, scale)
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl


def _check(o, lse, ro, rl, dtype):
    fin = np.isfinite(rl)
    assert np.isfinite(o).all() and np.array_equal(np.isfinite(lse), fin)
    assert np.all(o[~fin] == 0) and np.all(lse[~fin] == -np.inf)
    if dtype == torch.bfloat16:
        assert np.abs(o - ro).max() <= 2e-2
        assert np.abs(lse[fin] - rl[fin]).max(initial=0) <= 2e-2
    else:
        assert np.abs(o - ro).max() <= 1e-5 * np.abs(ro).max()
        assert np.abs(lse[fin] - rl[fin]).max(initial=0) <= 1e-5 * max(1, np.abs(rl).max())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bs,d", [(32, 64), (32, 128), (64, 64), (64, 128)])
def test_decode_int8_loglinear(dtype, bs, d):
    n_cap = 16 * bs
    lengths = [1, bs, bs + 1, n_cap // 2 + 5, n_cap - 1, n_cap]
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(n_cap, bs))
    o, lse, ro, rl = _decode_case(len(lengths), 2, n_cap, d, bs, dtype, lengths, mask, 3)
    _check(o, lse, ro, rl, dtype)


@pytest.mark.parametrize("bs,d", [(32, 64), (32, 128), (64, 64), (64, 128)])
def test_decode_int8_garbage_after_the_token(bs, d):
    # after each sequence's length: codes outside [-127, 127] (-128) and
    # random bytes in the token's own block, NaN scales in the blocks past it
    n_cap = 8 * bs
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(n_cap, bs))
    lengths = [1, 17, bs - 1, bs + 1, 3 * bs - 1, 5 * bs + 9, n_cap]
    B, H = len(lengths), 2
    q = _randn((B, H, d), torch.bfloat16, 21 + d)
    k = _randn((B, H, n_cap, d), torch.float32, 22 + d)
    v = _randn((B, H, n_cap, d), torch.float32, 23 + d)
    kc, ks = oracle.quantize_blocks(k.numpy(), bs)
    vc, vs = oracle.quantize_blocks(v.numpy(), bs)
    ro, rl = oracle.block_sparse_decode_int8(q.double().numpy(), kc, ks, vc, vs, lengths, mask, bs)
    rng = np.random.default_rng(bs + d)
    kc, vc, ks, vs = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    for b, L in enumerate(lengths):
        kc[b, :, L:] = rng.integers(-128, 128, kc[b, :, L:].shape, dtype=np.int8)
        vc[b, :, L:] = -128
        first_past = -(-L // bs)  # blocks wholly after the token
        ks[b, :, first_past:] = np.nan
        vs[b, :, first_past:] = np.inf
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(n_cap, bs, mask=mask)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, lse = bsa.decode_int8kv(q.to(dev), t(kc), t(ks), t(vc), t(vs),
                               torch.tensor(lengths, dtype=torch.int32, device=dev),
                               rp.to(dev), ci.to(dev), bs)
    torch.cuda.synchronize()
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("q_scale", [2.0 ** 14, 2.0 ** -20])
def test_decode_int8_query_magnitudes(d, q_scale):
    # a bf16 query far outside float16 range (2^14 N(0,1): |q| up to ~2^16)
    # and one far below its normal range; the scores' float16 form scales q
    # by a power of two, which must not show in the result
    bs, n_cap = 32, 512
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(n_cap, bs))
    lengths = [n_cap, 300, 45]
    B, H = len(lengths), 2
    q = (_randn((B, H, d), torch.float32, 31) * q_scale).to(torch.bfloat16)
    k = _randn((B, H, n_cap, d), torch.float32, 32)
    v = _randn((B, H, n_cap, d), torch.float32, 33)
    kc, ks = oracle.quantize_blocks(k.numpy(), bs)
    vc, vs = oracle.quantize_blocks(v.numpy(), bs)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(n_cap, bs)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, lse = bsa.decode_int8kv(q.to(dev), t(kc), t(ks), t(vc), t(vs),
                               torch.tensor(lengths, dtype=torch.int32, device=dev),
                               rp.to(dev), ci.to(dev), bs)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_decode_int8(q.double().numpy(), kc, ks, vc, vs, lengths, mask, bs)
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.abs(o - ro).max() <= 2e-2
    # the LSE is as large as the scores: float32 relative accuracy
    assert np.abs(lse - rl).max() <= 2e-2 * max(1.0, 1e-3 * np.abs(rl).max())


def test_decode_int8_random_mask_per_head_and_scale():
    bs, d, n_cap, H = 32, 64, 1024, 3
    M = n_cap // bs
    masks = [random_block_mask(M, 0.2 + 0.2 * h, 40 + h) for h in range(H)]
    lengths = [1000, 17, 512, 1024, 33]
    o, lse, ro, rl = _decode_case(len(lengths), H, n_cap, d, bs, torch.bfloat16, lengths, masks,
                                  7, per_head=True, scale=0.3)
    _check(o, lse, ro, rl, torch.bfloat16)


def test_decode_int8_worked_example_cache_full_size():
    # B=32 sequences on the worked example's cache (N=4096, d=64, block 32, log-linear),
    # mixed lengths; sampled (b, h) checked against the oracle
    B, H, N, d, bs = 32, 8, 4096, 64, 32
    dev = torch.device("cuda")
    q = _randn((B, H, d), torch.bfloat16, 1)
    k = _randn((B, H, N, d), torch.bfloat16, 2)
    v = _randn((B, H, N, d), torch.bfloat16, 3)
    kc, ks = bsa.quantize_kv(k.to(dev), bs)
    vc, vs = bsa.quantize_kv(v.to(dev), bs)
    lengths = torch.from_numpy(np.random.default_rng(5).integers(1, N + 1, B).astype(np.int32))
    rp, ci = bsa.build_pattern(N, bs)
    o, lse = bsa.decode_int8kv(q.to(dev), kc, ks, vc, vs, lengths.to(dev), rp.to(dev),
                               ci.to(dev), bs)
    torch.cuda.synchronize()
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    for b, h in ((0, 0), (5, 3), (31, 7), (20, 1)):
        # oracle codes from the oracle quantiser (the GPU's are checked bit-exact above)
        rkc, rks = oracle.quantize_blocks(k[b, h].float().numpy(), bs)
        rvc, rvs = oracle.quantize_blocks(v[b, h].float().numpy(), bs)
        ro, rl = oracle.block_sparse_decode_head(
            q[b, h].double().numpy(), oracle.dequantize_blocks(rkc, rks, bs),
            oracle.dequantize_blocks(rvc, rvs, bs), int(lengths[b]), mask, bs)
        assert np.abs(o[b, h].double().cpu().numpy() - ro).max() <= 2e-2
        assert abs(lse[b, h].item() - rl) <= 2e-2
