"""GPU parity of the forward variants: causal masking, one pattern per head,
and the dilated-window and BigBird patterns, all through the C ABI
(bsa_forward_ex) against the float64 oracle."""

import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from workgroup_shapes import runnable_cases
from synthetic_inputs import WORKLOADS, make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

BF16_ATOL = 2e-2
F32_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa._load()


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _compare(o, lse, o_ref, lse_ref, dtype, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"non-finite output {what}"
    if dtype == torch.float32:
        eo = np.abs(o - o_ref).max() / np.abs(o_ref).max()
        el = np.abs(lse - lse_ref).max() / np.abs(lse_ref).max()
        assert eo <= F32_RTOL and el <= F32_RTOL, f"{what} rel err O {eo:.3e} LSE {el:.3e}"
    else:
        eo = np.abs(o - o_ref).max()
        el = np.abs(lse - lse_ref).max()
        assert eo <= 2e-2 and el <= 2e-2, f"{what} abs err O {eo:.3e} LSE {el:.3e}"
    return eo, el


def _sets(kind, N, bs, seed):
    M = N // bs
    if kind == "loglinear":
        return oracle.loglinear_block_sets(N, bs), {}
    if kind == "ones":
        return [set(range(M)) for _ in range(M)], {"mask": np.ones((M, M), np.uint8)}
    if kind == "random":
        m = random_block_mask(M, 0.4, seed)
        return [set(np.nonzero(m[i])[0].tolist()) for i in range(M)], {"mask": m}
    if kind == "dilated":
        return (oracle.dilated_block_sets(N, bs, window=2, dilation=3, global_blocks=[0]),
                {"kind": "dilated", "window": 2, "dilation": 3, "global_blocks": [0]})
    if kind == "bigbird":
        return (oracle.bigbird_block_sets(N, bs, num_random=2, seed=seed, global_blocks=[0]),
                {"kind": "bigbird", "num_random": 2, "seed": seed, "global_blocks": [0]})
    raise ValueError(kind)


CASES = [(dt, bs, d, kind, B, H, M)
         for dt in ("bf16", "f32") for bs in (32, 64) for d in (64, 128)
         for kind, B, H, M in (("loglinear", 1, 2, 9), ("ones", 2, 1, 5), ("random", 1, 3, 7),
                               ("dilated", 1, 2, 11), ("bigbird", 2, 2, 10))]


@pytest.mark.parametrize("dt,bs,d,kind,B,H,M", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_variant_parity(dt, bs, d, kind, B, H, M, causal):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    N = bs * M
    seed = zlib.crc32(repr((dt, bs, d, kind, B, H, M, causal)).encode()) % 1000
    q, k, v = make_qkv(B, H, N, d, dtype, seed)
    sets, kw = _sets(kind, N, bs, seed)
    if causal:
        sets = oracle.causal_block_sets(sets)
    mask = oracle.block_mask_from_sets(sets)
    rp, ci = bsa.build_pattern(N, bs, causal=causal, **kw)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs,
                                                   causal=causal)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, dtype, f"{dt} bs{bs} d{d} {kind} causal={causal}")


@pytest.mark.parametrize("dt,bs,d,group,key_split",
                         runnable_cases([("bf16", 32, 64), ("bf16", 64, 128)]))
def test_causal_on_a_non_causal_pattern_every_shape(dt, bs, d, group, key_split):
    """The kernel itself skips blocks after the query block and masks the
    diagonal block: a pattern that still holds j > i gives the causal result."""
    B, H, M = 2, 2, 11
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 31)
    m = random_block_mask(M, 0.5, 31)
    rp, ci = bsa.build_pattern(N, bs, mask=m)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         causal=True, group=group, key_split=key_split)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), m, bs, causal=True)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, torch.bfloat16, f"G{group} KS{key_split}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt,bs,d", [("bf16", 32, 64), ("bf16", 64, 128), ("f32", 64, 64)])
def test_per_head_patterns(dt, bs, d, causal):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 4, 12
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, dtype, 41)
    kinds = ["loglinear", "dilated", "bigbird", "random"]
    pats, masks = [], []
    for h, kind in enumerate(kinds):
        sets, kw = _sets(kind, N, bs, 100 + h)
        if causal:
            sets = oracle.causal_block_sets(sets)
        pats.append(bsa.build_pattern(N, bs, causal=causal, **kw))
        masks.append(oracle.block_mask_from_sets(sets))
    rp, ci = bsa.stack_head_patterns(pats)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         causal=causal, per_head=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), np.stack(masks), bs,
                                                   causal=causal)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, dtype, f"per-head {dt} bs{bs} d{d}")


def test_causal_worked_example_sampled():
    w = WORKLOADS["worked_example"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, 0)
    rp, ci = bsa.build_pattern(w.N, w.block_size, causal=True)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), w.block_size,
                         causal=True)
    torch.cuda.synchronize()
    sets = oracle.causal_block_sets(oracle.loglinear_block_sets(w.N, w.block_size))
    mask = oracle.block_mask_from_sets(sets)
    assert int(rp[-1]) == int(mask.sum())
    for h in (0, 5):
        o_ref, lse_ref = oracle.block_sparse_attention_head(
            _f64(q[0, h]), _f64(k[0, h]), _f64(v[0, h]), mask, w.block_size,
            query_blocks=[0, 1, 2, 63, 64, 65, 126, 127], causal=True)
        rows = np.isfinite(lse_ref)
        _compare(_f64(o[0, h])[rows], _f64(lse[0, h])[rows], o_ref[rows], lse_ref[rows],
                 torch.bfloat16, f"causal worked example h{h}")
