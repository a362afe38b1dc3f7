"""The Python binding checks every caller-supplied device buffer and the
pattern arrays' sizes before it calls the C ABI (which takes raw pointers and
cannot see a too-small buffer).  Each case raises before any launch."""

import pytest
import torch

import block_sparse_attention_csr_amd as bsa
from synthetic_inputs import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _setup(dev, B=1, H=2, M=4, bs=32, d=64):
    q, k, v = (t.to(dev) for t in make_qkv(B, H, M * bs, d, torch.bfloat16, 3))
    rp, ci = bsa.build_pattern(M * bs, bs)
    return q, k, v, rp.to(dev), ci.to(dev), bs


def test_forward_rejects_bad_buffers(dev):
    q, k, v, rp, ci, bs = _setup(dev)
    B, H, N, d = q.shape
    bad = [
        dict(out=torch.empty((B, H, N - 1, d), dtype=q.dtype, device=dev)),
        dict(out=torch.empty_like(q, dtype=torch.float32)),
        dict(out=torch.empty((B, H, d, N), dtype=q.dtype, device=dev).transpose(2, 3)),
        dict(lse=torch.empty((B, H, N), dtype=torch.bfloat16, device=dev)),
        dict(lse=torch.empty((B, H, N - 32), dtype=torch.float32, device=dev)),
        dict(nnz=ci.numel() + 1),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            bsa.forward(q, k, v, rp, ci, bs, **kw)
    with pytest.raises(ValueError):  # row_ptr of another block count
        bsa.forward(q, k, v, rp[:-1], ci, bs)
    with pytest.raises(ValueError):  # per-head flag with one shared pattern
        bsa.forward(q, k, v, rp, ci, bs, per_head=True)
    o, lse = bsa.forward(q, k, v, rp, ci, bs)  # the same call with good buffers runs
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_backward_rejects_bad_buffers(dev):
    q, k, v, rp, ci, bs = _setup(dev)
    cp, ri = bsa.transpose_pattern(rp.cpu(), ci.cpu())
    cp, ri = cp.to(dev), ri.to(dev)
    o, lse = bsa.forward(q, k, v, rp, ci, bs)
    B, H, N, d = q.shape
    args = (q, k, v, o, lse, torch.randn_like(q), rp, ci, cp, ri, bs)
    for kw in (dict(dq=torch.empty((B, H, N, d // 2), dtype=q.dtype, device=dev)),
               dict(delta=torch.empty((B, H, N), dtype=torch.bfloat16, device=dev))):
        with pytest.raises(ValueError):
            bsa.backward(*args, **kw)
    with pytest.raises(ValueError):  # lse of the wrong shape
        bsa.backward(q, k, v, o, lse[:, :1], torch.randn_like(q), rp, ci, cp, ri, bs)
    with pytest.raises(ValueError):  # CSC offsets of another size
        bsa.backward(q, k, v, o, lse, torch.randn_like(q), rp, ci, cp[:-1], ri, bs)
    torch.cuda.synchronize()


def test_decode_and_quantiser_reject_bad_buffers(dev):
    B, H, n_cap, d, bs = 2, 2, 128, 64, 32
    q = torch.randn(B, H, d, device=dev).bfloat16()
    kc = torch.randn(B, H, n_cap, d, device=dev).bfloat16()
    vc = torch.randn(B, H, n_cap, d, device=dev).bfloat16()
    sl = torch.tensor([5, 100], dtype=torch.int32, device=dev)
    rp, ci = (t.to(dev) for t in bsa.build_pattern(n_cap, bs))
    with pytest.raises(ValueError):
        bsa.decode(q, kc, vc, sl.long(), rp, ci, bs)
    with pytest.raises(ValueError):
        bsa.decode(q, kc, vc, sl, rp, ci, bs, out=torch.empty((B, H, d + 1), device=dev))
    with pytest.raises(ValueError):
        bsa.decode(q, kc, vc, sl, rp, ci, bs, lse=torch.empty((B,), device=dev))
    with pytest.raises(ValueError):
        bsa.quantize_kv(kc, bs, codes=torch.empty((B, H, n_cap, d), dtype=torch.uint8,
                                                  device=dev))
    with pytest.raises(ValueError):
        bsa.quantize_kv(kc, bs, scales=torch.empty((B, H, n_cap), device=dev))
    k8, ks = bsa.quantize_kv(kc, bs)
    v8, vs = bsa.quantize_kv(vc, bs)
    with pytest.raises(ValueError):
        bsa.decode_int8kv(q, k8, ks[:, :, :-1], v8, vs, sl, rp, ci, bs)
    with pytest.raises(ValueError):
        bsa.decode_int8kv(q, k8, ks, v8, vs, sl, rp[:-1], ci, bs)
    od, ld = bsa.decode_int8kv(q, k8, ks, v8, vs, sl, rp, ci, bs)
    torch.cuda.synchronize()
    assert torch.isfinite(od.float()).all() and torch.isfinite(ld).all()


def test_side_stream_scratch_is_not_reused_early(dev):
    """forward(split=...) and backward enqueued on a side stream while the
    current stream keeps allocating and writing: the binding allocates the
    row-split workspace, delta and the outputs on the side stream, so the
    caching allocator cannot hand them to the current stream's work while the
    side stream's kernels still use them.  Results match the oracle."""
    import numpy as np

    import oracle
    from synthetic_inputs import local_global_block_mask

    B, H, M, bs, d = 2, 2, 16, 64, 128
    N = M * bs
    mask = local_global_block_mask(M)
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 5)
    g = make_qkv(B, H, N, d, torch.bfloat16, 6)[0]
    rp, ci = bsa.build_pattern(N, bs, mask=mask)
    cp, ri = bsa.transpose_pattern(rp, ci)
    plan = bsa.plan_row_split(rp, 4)
    assert plan is not None
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    rpd, cid, cpd, rid = (t.to(dev) for t in (rp, ci, cp, ri))
    pland = plan.to(dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    # hold the side stream so its kernels are still queued when the
    # function returns and the temporaries it allocated are dropped
    with torch.cuda.stream(side):
        torch.cuda._sleep(int(5e7))
    o, lse = bsa.forward(qd, kd, vd, rpd, cid, bs, split=pland, stream=side)
    dq, dk, dv = bsa.backward(qd, kd, vd, o, lse, gd, rpd, cid, cpd, rid, bs, stream=side)
    # the current stream meanwhile allocates and overwrites fresh memory
    junk = [torch.full((1 << 20,), float("nan"), device=dev) for _ in range(64)]
    torch.cuda.synchronize()
    del junk
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.block_sparse_attention(f(q), f(k), f(v), mask, bs)
    assert np.abs(f(o) - o_ref).max() <= 2e-2 and np.abs(f(lse) - lse_ref).max() <= 2e-2
    ref = oracle.block_sparse_attention_backward(f(q), f(k), f(v), f(g), mask, bs)
    for got, want in zip((dq, dk, dv), ref[:3]):
        assert np.abs(f(got) - want).max() <= 2e-2 * max(1.0, float(np.abs(want).max()))
