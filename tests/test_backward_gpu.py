"""GPU parity of the backward (bsa_backward through the C ABI) against the
float64 oracle: dQ, dK, dV for every dtype, block size and head size, plain
and causal, on log-linear, random and all-ones patterns."""

import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import WORKLOADS, make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

# bf16: P and dS are rounded to bf16 before their products (as in the
# forward), so the bound is relative to the gradient's magnitude:
# max|err| <= 2e-2 * max(1, max|ref|).  fp32: max|err| <= 1e-4 * max|ref|.
BF16_TOL = 2e-2
F32_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa._load()


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, got, ref, dtype):
    got = _f64(got)
    assert np.isfinite(got).all(), f"{name}: non-finite gradient"
    err = np.abs(got - ref).max()
    mag = np.abs(ref).max()
    if dtype == torch.float32:
        assert err <= F32_TOL * mag, f"{name}: max err {err:.3e} vs max |ref| {mag:.3e}"
    else:
        assert err <= BF16_TOL * max(1.0, mag), f"{name}: max err {err:.3e} vs max |ref| {mag:.3e}"
    return err / max(1.0, mag)


def _mask(kind, M, seed):
    if kind == "loglinear":
        return oracle.block_mask_from_sets(oracle.loglinear_block_sets(M * 32, 32)), None
    if kind == "ones":
        m = np.ones((M, M), np.uint8)
    else:
        m = random_block_mask(M, 0.4, seed)
    return m, m


def _run(q, k, v, do, bs, user_mask, causal, scale=None):
    """Backward with the longest-first block orders, checked to give exactly
    the result of the ascending order (the order only schedules the work)."""
    dev = torch.device("cuda")
    N = q.shape[2]
    rp, ci = bsa.build_pattern(N, bs, mask=user_mask, causal=causal)
    cp, ri = bsa.transpose_pattern(rp, ci)
    ro, co = bsa.pattern_order(rp), bsa.pattern_order(cp)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    rp, ci, cp, ri, ro, co = (t.to(dev) for t in (rp, ci, cp, ri, ro, co))
    o, lse = bsa.forward(q, k, v, rp, ci, bs, scale, causal=causal)
    dq, dk, dv = bsa.backward(q, k, v, o, lse, do, rp, ci, cp, ri, bs, scale, causal=causal,
                              row_order=ro, col_order=co)
    plain = bsa.backward(q, k, v, o, lse, do, rp, ci, cp, ri, bs, scale, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), plain):
        assert torch.equal(a, b)
    return dq, dk, dv


CASES = [(dt, bs, d, kind, B, H, M) for dt in ("bf16", "f32") for bs in (32, 64)
         for d in (64, 128)
         for kind, B, H, M in (("loglinear", 1, 2, 9), ("random", 2, 1, 7), ("ones", 1, 1, 5))]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt,bs,d,kind,B,H,M", CASES)
def test_backward_parity(dt, bs, d, kind, B, H, M, causal):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    N = bs * M
    seed = zlib.crc32(repr((dt, bs, d, kind, B, H, M, causal)).encode()) % 1000
    q, k, v = make_qkv(B, H, N, d, dtype, seed)
    do = make_qkv(B, H, N, d, dtype, seed + 1)[0]
    if kind == "loglinear":
        sets = oracle.loglinear_block_sets(N, bs)
        mask, user = oracle.block_mask_from_sets(sets), None
    else:
        mask, user = _mask(kind, M, seed)
    if causal:
        mask = np.tril(mask)
    dq, dk, dv = _run(q, k, v, do, bs, user, causal)
    rq, rk, rv, _ = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do),
                                                           mask, bs, causal=causal)
    what = f"{dt} bs{bs} d{d} {kind} causal={causal}"
    _check(f"dQ {what}", dq, rq, dtype)
    _check(f"dK {what}", dk, rk, dtype)
    _check(f"dV {what}", dv, rv, dtype)


@pytest.mark.parametrize("dt,bs,d", [(dt, bs, d) for dt in ("bf16", "f32") for bs in (32, 64)
                                     for d in (64, 128)])
def test_backward_key_blocks_no_query_selects(dt, bs, d):
    """Empty CSC columns: every query block selects only blocks 0 and M - 1
    (and its own for M - 2), so most key blocks are selected by no query:
    their dK and dV are exactly 0."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 2, 7
    N = bs * M
    m = np.zeros((M, M), np.uint8)
    m[:, 0] = 1
    m[:, M - 1] = 1
    m[M - 2, M - 2] = 1
    q, k, v = make_qkv(B, H, N, d, dtype, 61)
    do = make_qkv(B, H, N, d, dtype, 62)[0]
    dq, dk, dv = _run(q, k, v, do, bs, m, False)
    rq, rk, rv, _ = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do),
                                                           m, bs)
    for j in range(1, M - 2):  # no query block selects key block j
        sl = slice(j * bs, (j + 1) * bs)
        assert torch.all(dk[:, :, sl] == 0) and torch.all(dv[:, :, sl] == 0)
    what = f"{dt} bs{bs} d{d} empty columns"
    _check(f"dQ {what}", dq, rq, dtype)
    _check(f"dK {what}", dk, rk, dtype)
    _check(f"dV {what}", dv, rv, dtype)


def test_backward_scale_override():
    q, k, v = make_qkv(1, 2, 64 * 6, 64, torch.bfloat16, 5)
    do = make_qkv(1, 2, 64 * 6, 64, torch.bfloat16, 6)[0]
    m = random_block_mask(6, 0.5, 5)
    dq, dk, dv = _run(q, k, v, do, 64, m, False, scale=0.3)
    rq, rk, rv, _ = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do),
                                                           m, 64, scale=0.3)
    for name, a, b in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        _check(name, a, b, torch.bfloat16)


def test_backward_worked_example_sampled_heads():
    w = WORKLOADS["worked_example"]
    q, k, v = make_qkv(1, 2, w.N, w.d, w.torch_dtype, 0)
    do = make_qkv(1, 2, w.N, w.d, w.torch_dtype, 1)[0]
    dq, dk, dv = _run(q, k, v, do, w.block_size, None, False)
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(w.N, w.block_size))
    rq, rk, rv, _ = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do),
                                                           mask, w.block_size)
    for name, a, b in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        print(name, _check(name, a, b, torch.bfloat16))


def test_backward_deterministic():
    q, k, v = make_qkv(2, 2, 1024, 64, torch.bfloat16, 3)
    do = make_qkv(2, 2, 1024, 64, torch.bfloat16, 4)[0]
    a = _run(q, k, v, do, 32, None, False)
    b = _run(q, k, v, do, 32, None, False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_wrapper_matches_the_oracle():
    """bsa.attention as a torch.autograd.Function: O from the forward kernel,
    gradients from the backward kernels, checked against the oracle."""
    bs, d, M, B, H = 32, 64, 12, 2, 2
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 41)
    g = make_qkv(B, H, N, d, torch.bfloat16, 42)[0]
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs)
    cp, ri = bsa.transpose_pattern(rp, ci)
    ro, co = bsa.pattern_order(rp).to(dev), bsa.pattern_order(cp).to(dev)
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    o = bsa.attention(qd, kd, vd, rp.to(dev), ci.to(dev), cp.to(dev), ri.to(dev), bs,
                      row_order=ro, col_order=co)
    (o.float() * g.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    o_ref, _ = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs)
    assert np.abs(_f64(o.detach()) - o_ref).max() <= 2e-2
    rq, rk, rv, _ = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(g),
                                                           mask, bs)
    _check("dQ autograd", qd.grad, rq, torch.bfloat16)
    _check("dK autograd", kd.grad, rk, torch.bfloat16)
    _check("dV autograd", vd.grad, rv, torch.bfloat16)


def test_backward_largest_block_count_invariants():
    """M = 4096 blocks (N = 131072 at block 32, the largest the backward
    takes): properties that hold at any size, since every softmax row sums to
    one and every row of dS sums to zero:
      sum over keys of dV = sum over queries of dO,
      sum over keys of dK = 0,
    per (batch, head) and feature; plus finite gradients everywhere."""
    B, H, N, d, bs = 1, 2, 131072, 64, 32
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 8)
    do = make_qkv(B, H, N, d, torch.bfloat16, 9)[0]
    dq, dk, dv = _run(q, k, v, do, bs, None, False)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    sum_dv = dv.double().sum(dim=2)
    sum_do = do.double().sum(dim=2).to(sum_dv.device)
    e_dv = (sum_dv - sum_do).abs().max().item()
    e_dk = dk.double().sum(dim=2).abs().max().item()
    print(f"M=4096 invariants: max |sum dV - sum dO| {e_dv:.3e}, max |sum dK| {e_dk:.3e}, "
          f"max |sum dO| {sum_do.abs().max().item():.3e}")
    # Each gradient element carries a bf16 rounding of relative size up to
    # 2^-8 on values of magnitude ~1, with random signs: over N terms the sum
    # drifts by ~2^-8 sqrt(N) (1.4 here; measured 0.2).  One missing 32-row key
    # block would move the sums by ~32.
    tol = 2.0 ** -8 * N ** 0.5
    assert e_dv <= tol
    assert e_dk <= tol


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt,bs,d", [("bf16", 32, 64), ("bf16", 64, 128), ("f32", 64, 64)])
def test_backward_per_head_patterns(dt, bs, d, causal):
    """One pattern per head (the log-linear page's section 2.2 speaks of
    per-head patterns): row_ptr and col_ptr are [H, M + 1], each head's CSC
    the transpose of its CSR; dQ, dK, dV against the oracle with [H, M, M]
    masks, through bsa_backward and bsa_backward_noalloc."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 4, 10
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, dtype, 91)
    do = make_qkv(B, H, N, d, dtype, 92)[0]
    masks = [random_block_mask(M, 0.3 + 0.15 * h, 93 + h) for h in range(H)]
    csrs = [bsa.build_pattern(N, bs, mask=m, causal=causal) for m in masks]
    cscs = [bsa.transpose_pattern(rp, ci) for rp, ci in csrs]
    rp, ci = bsa.stack_head_patterns(csrs)
    cp, ri = bsa.stack_head_patterns(cscs)
    dev = torch.device("cuda")
    t = [x.to(dev) for x in (q, k, v, do)]
    pat = [x.to(dev) for x in (rp, ci, cp, ri)]
    o, lse = bsa.forward(t[0], t[1], t[2], pat[0], pat[1], bs, causal=causal, per_head=True)
    grads = bsa.backward(t[0], t[1], t[2], o, lse, t[3], *pat, bs, causal=causal, per_head=True)
    out = [torch.empty_like(t[0]) for _ in range(3)]
    grads2 = bsa.backward_noalloc(t[0], t[1], t[2], o, lse, t[3], *pat, bs, *out, causal=causal,
                                  per_head=True)
    torch.cuda.synchronize()
    ref = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do),
                                                 np.stack(masks), bs, causal=causal)
    for name, got, want, again in zip(("dQ", "dK", "dV"), grads, ref[:3], grads2):
        _check(f"{name} {dt} bs{bs} d{d} causal={causal}", got, want, dtype)
        assert torch.equal(got, again), name
    with pytest.raises(ValueError):  # orders are of one shared pattern
        bsa.backward(t[0], t[1], t[2], o, lse, t[3], *pat, bs, per_head=True,
                     row_order=torch.zeros(M, dtype=torch.int32, device=dev))


def test_backward_more_than_4096_blocks_sampled():
    """M = 8192 query blocks (N = 262144 at block 32), beyond what an LDS entry
    list held: a banded pattern of independent groups of four blocks, so that
    the gradients of the tokens of one group equal the dense backward of that
    128-token segment alone.  Sampled groups (first, middle, last) against
    the oracle on their segment."""
    B, H, d, bs, M = 1, 1, 64, 32, 8192
    N = M * bs
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 97)
    do = make_qkv(B, H, N, d, torch.bfloat16, 98)[0]
    i = np.arange(M)
    rows = [list(range(4 * (r // 4), 4 * (r // 4) + 4)) for r in range(M)]
    rp = torch.tensor(np.concatenate([[0], np.cumsum([len(r) for r in rows])]), dtype=torch.int32)
    ci = torch.tensor([j for r in rows for j in r], dtype=torch.int32)
    cp, ri = bsa.transpose_pattern(rp, ci)
    dev = torch.device("cuda")
    t = [x.to(dev) for x in (q, k, v, do)]
    pat = [x.to(dev) for x in (rp, ci, cp, ri)]
    o, lse = bsa.forward(t[0], t[1], t[2], pat[0], pat[1], bs)
    dq, dk, dv = bsa.backward(t[0], t[1], t[2], o, lse, t[3], *pat, bs)
    torch.cuda.synchronize()
    assert len(i) == M
    ones = np.ones((4, 4), np.uint8)
    for g in (0, 1, M // 8, M // 4 - 1):
        seg = slice(g * 128, (g + 1) * 128)
        f = lambda x: _f64(x[:, :, seg])
        ref = oracle.block_sparse_attention_backward(f(q), f(k), f(v), f(do), ones, bs)
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref[:3]):
            _check(f"{name} group {g}", got[:, :, seg], want, torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind,causal", [("loglinear", False), ("loglinear", True),
                                         ("random", False), ("random", True)])
def test_backward_grouped_blocks_sampled_heads(kind, causal, d):
    """Block 32 on a large grid (B H M = 16384 query blocks): four query
    blocks per dQ workgroup share each K/V stage of the union of their rows
    (the dK/dV kernel takes one key block per workgroup).  Sampled heads
    against the oracle on those heads (every head is independent), and the
    same result as the ascending order."""
    B, H, bs, M = 16, 8, 32, 128
    N = M * bs
    seed = zlib.crc32(repr(("grouped", kind, causal, d)).encode()) % 1000
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed)
    do = make_qkv(B, H, N, d, torch.bfloat16, seed + 1)[0]
    if kind == "loglinear":
        mask, user = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs)), None
    else:
        mask, user = _mask(kind, M, seed)
    if causal:
        mask = np.tril(mask)
    dq, dk, dv = _run(q, k, v, do, bs, user, causal)
    for b, h in ((0, 0), (7, 3), (B - 1, H - 1)):
        f = lambda x: _f64(x[b:b + 1, h:h + 1])
        ref = oracle.block_sparse_attention_backward(f(q), f(k), f(v), f(do), mask, bs,
                                                     causal=causal)
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref[:3]):
            _check(f"{name} ({b}, {h}) {kind} causal={causal} d{d}", got[b:b + 1, h:h + 1],
                   want, torch.bfloat16)


@pytest.mark.parametrize("which", ["rows", "columns"])
def test_backward_more_than_64_long_blocks(which):
    """70 of M = 160 blocks are long (more than twice the mean entry count):
    the kernels count the long blocks of a work order 64 at a time, so this
    count spans two chunks.  "rows": query blocks 0..69 select every key
    block, the others their own; "columns": the transpose, key blocks 0..69
    selected by every query block.  On a grid large enough for grouped dQ
    workgroups (B H M = 10240); the ordered result must equal the ascending
    one bit for bit (a miscounted prefix would drop or repeat blocks), and
    sampled heads match the oracle."""
    B, H, bs, d, M, L = 8, 8, 32, 64, 160, 70
    N = M * bs
    mask = np.zeros((M, M), np.uint8)
    if which == "rows":
        mask[:L, :] = 1
    else:
        mask[:, :L] = 1
    np.fill_diagonal(mask, 1)
    counts = mask.sum(axis=1 if which == "rows" else 0)
    assert int((counts * M > 2 * counts.sum()).sum()) == L
    seed = zlib.crc32(repr(("long blocks", which)).encode()) % 1000
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed)
    do = make_qkv(B, H, N, d, torch.bfloat16, seed + 1)[0]
    dq, dk, dv = _run(q, k, v, do, bs, mask, False)
    for b, h in ((0, 0), (B - 1, H - 1)):
        f = lambda x: _f64(x[b:b + 1, h:h + 1])
        ref = oracle.block_sparse_attention_backward(f(q), f(k), f(v), f(do), mask, bs)
        for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref[:3]):
            _check(f"{name} ({b}, {h}) long {which}", got[b:b + 1, h:h + 1], want,
                   torch.bfloat16)
