"""The forward on int8 K/V with one scale per block (bsa_forward_int8kv
through the C ABI) against the float64 oracle on the dequantised values
(codes * scales: the log-linear page's section 6.3 keeps K/V in int8 and
computes attention in 16-bit floating point).  Codes and scales come from
the oracle's quantiser; the bar is the bf16 one (max-abs 2e-2 on O and LSE).
Every workgroup shape, causal masking, per-head patterns, rows with no or
out-of-range entries, all-zero blocks (scale 0) and the worked example at
full size."""

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import make_qkv, random_block_mask
from workgroup_shapes import runnable_cases

pytestmark = pytest.mark.gpu

CONFIGS = [("bf16", 32, 64), ("bf16", 32, 128), ("bf16", 64, 64), ("bf16", 64, 128)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _quantized(k, v, bs):
    """Oracle codes and scales of K and V, and their float64 dequantisation."""
    kq, ks = oracle.quantize_blocks(_f64(k), bs)
    vq, vs = oracle.quantize_blocks(_f64(v), bs)
    kd = oracle.dequantize_blocks(kq, ks, bs)
    vd = oracle.dequantize_blocks(vq, vs, bs)
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return (t(kq), t(ks), t(vq), t(vs)), kd, vd


def _check(o, lse, o_ref, lse_ref, what, rows=None):
    o, lse = _f64(o), _f64(lse)
    if rows is not None:
        o, lse, o_ref, lse_ref = o[..., rows, :], lse[..., rows], o_ref[..., rows, :], lse_ref[..., rows]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), what
    assert np.abs(o - o_ref).max() <= 2e-2, (what, np.abs(o - o_ref).max())
    assert np.abs(lse - lse_ref).max() <= 2e-2, (what, np.abs(lse - lse_ref).max())


@pytest.mark.parametrize("dt,bs,d,group,key_split", runnable_cases(CONFIGS) + [
    ("bf16", 32, 64, 0, 0), ("bf16", 64, 128, 0, 0)])
def test_int8kv_every_workgroup_shape(dt, bs, d, group, key_split):
    B, H, M = 2, 3, 11
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 51)
    mask = random_block_mask(M, 0.4, 51)
    (kq, ks, vq, vs), kd, vd = _quantized(k, v, bs)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs, mask=mask)
    o, lse = bsa.forward_int8kv(q.to(dev), kq, ks, vq, vs, rp.to(dev), ci.to(dev), bs,
                                group=group, key_split=key_split)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), kd, vd, mask, bs)
    _check(o, lse, o_ref, lse_ref, f"bs{bs} d{d} G{group} KS{key_split}")


@pytest.mark.parametrize("group,key_split", [(0, 0), (1, 1), (1, 2), (4, 1)])
@pytest.mark.parametrize("per_head", [False, True])
def test_int8kv_causal_and_per_head(group, key_split, per_head):
    bs, d, B, H, M = 32, 64, 2, 2, 12
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 61)
    masks = [random_block_mask(M, 0.5, 61 + h) for h in range(H)] if per_head else None
    (kq, ks, vq, vs), kd, vd = _quantized(k, v, bs)
    dev = torch.device("cuda")
    if per_head:
        rp, ci = bsa.stack_head_patterns([bsa.build_pattern(N, bs, mask=m, causal=True)
                                          for m in masks])
        mask = np.stack(masks)
    else:
        mask = random_block_mask(M, 0.5, 61)
        rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=True)
    o, lse = bsa.forward_int8kv(q.to(dev), kq, ks, vq, vs, rp.to(dev), ci.to(dev), bs,
                                causal=True, per_head=per_head, group=group, key_split=key_split)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), kd, vd, mask, bs, causal=True)
    _check(o, lse, o_ref, lse_ref, f"G{group} KS{key_split} per_head={per_head}")


@pytest.mark.parametrize("group,key_split", [(0, 0), (1, 2), (4, 1)])
def test_int8kv_zero_blocks_and_hand_made_csr(group, key_split):
    """All-zero K and V blocks (scale 0, codes 0) attend like any other
    (scores 0, values 0); a row with no entry and a row of out-of-range
    entries give O = 0 and LSE = -inf; out-of-range entries are skipped."""
    bs, d, B, H, M = 32, 64, 2, 2, 11
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 71)
    k[:, :, 3 * bs:4 * bs] = 0
    v[:, :, 5 * bs:6 * bs] = 0
    mask = random_block_mask(M, 0.45, 71)
    mask[:, 3] = 1
    mask[:, 5] = 1
    rows = [sorted(np.nonzero(mask[i])[0].tolist()) for i in range(M)]
    rows[2] = []
    rows[7] = [-1, M + 3]
    rows[8] = [-2] + rows[8] + [M]
    rp = torch.tensor(np.cumsum([0] + [len(r) for r in rows]), dtype=torch.int32)
    ci = torch.tensor([j for r in rows for j in r], dtype=torch.int32)
    (kq, ks, vq, vs), kd, vd = _quantized(k, v, bs)
    assert float(ks[0, 0, 3]) == 0.0 and float(vs[0, 0, 5]) == 0.0
    dev = torch.device("cuda")
    o, lse = bsa.forward_int8kv(q.to(dev), kq, ks, vq, vs, rp.to(dev), ci.to(dev), bs,
                                group=group, key_split=key_split)
    torch.cuda.synchronize()
    eff = np.zeros((M, M), np.uint8)
    for i, r in enumerate(rows):
        for j in r:
            if 0 <= j < M:
                eff[i, j] = 1
    dead = [i for i in range(M) if not eff[i].any()]
    assert dead == [2, 7]
    of, lf = _f64(o), _f64(lse)
    for i in dead:
        assert np.all(of[:, :, i * bs:(i + 1) * bs] == 0)
        assert np.all(lf[:, :, i * bs:(i + 1) * bs] == -np.inf)
        eff[i, i] = 1
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), kd, vd, eff, bs)
    live = np.concatenate([np.arange(i * bs, (i + 1) * bs) for i in range(M) if i not in dead])
    _check(o, lse, o_ref, lse_ref, f"G{group} KS{key_split}", rows=live)


def test_int8kv_worked_example_full():
    """The pages' worked example (B=1 H=8 N=4096 d=64 block 32, log-linear)
    on int8 K/V, every head and row against the oracle."""
    B, H, N, d, bs = 1, 8, 4096, 64, 32
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 0)
    (kq, ks, vq, vs), kd, vd = _quantized(k, v, bs)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs)
    o, lse = bsa.forward_int8kv(q.to(dev), kq, ks, vq, vs, rp.to(dev), ci.to(dev), bs)
    torch.cuda.synchronize()
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), kd, vd, mask, bs)
    _check(o, lse, o_ref, lse_ref, "worked example")


def test_int8kv_large_grid_sampled():
    """A grid large enough for the four-block workgroups (B=8 H=8 N=4096,
    block 32): sampled heads and query blocks against the oracle, and the
    GPU quantiser's codes giving the same output as the oracle's."""
    B, H, N, d, bs = 8, 8, 4096, 64, 32
    M = N // bs
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 3)
    (kq, ks, vq, vs), kd, vd = _quantized(k, v, bs)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs)
    qd = q.to(dev)
    o, lse = bsa.forward_int8kv(qd, kq, ks, vq, vs, rp.to(dev), ci.to(dev), bs)
    k8, k8s = bsa.quantize_kv(k.to(dev), bs)
    v8, v8s = bsa.quantize_kv(v.to(dev), bs)
    o2, lse2 = bsa.forward_int8kv(qd, k8, k8s, v8, v8s, rp.to(dev), ci.to(dev), bs)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    qblocks = [0, 1, 2, 31, 63, 64, 65, 100, M - 2, M - 1]
    for b, h in [(0, 0), (3, 5), (B - 1, H - 1)]:
        o_ref, lse_ref = oracle.block_sparse_attention_head(
            _f64(q[b, h]), kd[b, h], vd[b, h], mask, bs, query_blocks=qblocks)
        rows = np.isfinite(lse_ref)
        assert rows.sum() == len(qblocks) * bs
        _check(o[b, h], lse[b, h], o_ref, lse_ref, f"b{b} h{h}", rows=rows)
