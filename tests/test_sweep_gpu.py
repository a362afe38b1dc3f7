"""Seeded randomized parity sweep against the float64 oracle: forward cases
drawn over dtype, block and head size, batch, heads, ragged block counts,
mask density, causal masking, per-head patterns, scale and the workgroup
shape; backward and decode cases drawn the same way.  Each case is small
enough for the oracle to check every output; the seed names the case."""

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

SHAPES = [(0, 0), (0, 0), (1, 1), (1, 2), (1, 4), (2, 1), (4, 1), (2, 2)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _draw(seed):
    rng = np.random.default_rng(seed)
    c = dict(dtype=torch.bfloat16 if rng.random() < 0.7 else torch.float32,
             bs=int(rng.choice([32, 64])), d=int(rng.choice([64, 128])),
             B=int(rng.integers(1, 4)), H=int(rng.integers(1, 4)), M=int(rng.integers(1, 14)),
             causal=bool(rng.random() < 0.35), per_head=bool(rng.random() < 0.3),
             density=float(rng.uniform(0.05, 0.9)),
             scale=None if rng.random() < 0.6 else float(rng.uniform(0.03, 0.6)))
    c["shape"] = SHAPES[int(rng.integers(len(SHAPES)))]
    n_masks = c["H"] if c["per_head"] else 1
    c["masks"] = [random_block_mask(c["M"], c["density"], seed * 10 + h) for h in range(n_masks)]
    return c


def _check(got, want, dtype, what):
    got = np.asarray(got, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite pattern differs"
    if not fin.any():
        return
    err = np.abs(got[fin] - want[fin]).max()
    if dtype == torch.bfloat16:
        assert err <= 2e-2, f"{what}: max abs err {err:.3e}"
    else:
        rel = err / max(np.abs(want[fin]).max(), 1e-30)
        assert rel <= 1e-5, f"{what}: rel err {rel:.3e}"


def _pattern(c, N, causal):
    if c["per_head"]:
        return bsa.stack_head_patterns([bsa.build_pattern(N, c["bs"], mask=m, causal=causal)
                                        for m in c["masks"]])
    return bsa.build_pattern(N, c["bs"], mask=c["masks"][0], causal=causal)


@pytest.mark.parametrize("seed", range(120))
def test_forward_sweep(seed):
    c = _draw(seed)
    dtype, bs, d, B, H, M = c["dtype"], c["bs"], c["d"], c["B"], c["H"], c["M"]
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, dtype, 1000 + seed)
    rp, ci = _pattern(c, N, c["causal"])
    dev = torch.device("cuda")
    g, ks = c["shape"]
    args = (q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs, c["scale"])
    kw = dict(causal=c["causal"], per_head=c["per_head"])
    try:
        o, lse = bsa.forward(*args, group=g, key_split=ks, **kw)
    except bsa.BsaError as e:  # a forced shape this size cannot take: the library's own
        assert e.status == 2
        o, lse = bsa.forward(*args, **kw)
    torch.cuda.synchronize()
    mask = np.stack(c["masks"]) if c["per_head"] else c["masks"][0]
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs,
                                                   c["scale"], causal=c["causal"])
    what = f"seed {seed}: {c['dtype']} bs{bs} d{d} B{B} H{H} M{M} causal={c['causal']} " \
           f"per_head={c['per_head']} shape={c['shape']}"
    _check(_f64(o), o_ref, dtype, "O " + what)
    _check(_f64(lse), lse_ref, dtype, "LSE " + what)


@pytest.mark.parametrize("seed", range(120, 150))
def test_backward_sweep(seed):
    c = _draw(seed)
    dtype, bs, d, B, H, M = c["dtype"], c["bs"], c["d"], c["B"], c["H"], c["M"]
    N = bs * M
    mask = c["masks"][0]  # the backward takes one pattern for all heads
    q, k, v = make_qkv(B, H, N, d, dtype, 2000 + seed)
    do = make_qkv(B, H, N, d, dtype, 3000 + seed)[0]
    rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=c["causal"])
    cp, ri = bsa.transpose_pattern(rp, ci)
    dev = torch.device("cuda")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    rp, ci, cp, ri = (t.to(dev) for t in (rp, ci, cp, ri))
    o, lse = bsa.forward(qd, kd, vd, rp, ci, bs, c["scale"], causal=c["causal"])
    dq, dk, dv = bsa.backward(qd, kd, vd, o, lse, dod, rp, ci, cp, ri, bs, c["scale"],
                              causal=c["causal"])
    torch.cuda.synchronize()
    m = np.tril(mask) if c["causal"] else mask
    ref = oracle.block_sparse_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do), m, bs,
                                                 c["scale"], causal=c["causal"])
    what = f"seed {seed}: {c['dtype']} bs{bs} d{d} B{B} H{H} M{M} causal={c['causal']}"
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref[:3]):
        got, want = _f64(got), want
        err = np.abs(got - want).max()
        bound = (2e-2 * max(1.0, np.abs(want).max()) if dtype == torch.bfloat16
                 else 1e-5 * max(np.abs(want).max(), 1e-30))
        assert np.isfinite(got).all() and err <= bound, f"{name} {what}: err {err:.3e}"


@pytest.mark.parametrize("seed", range(200, 240))
def test_decode_sweep(seed):
    c = _draw(seed)
    dtype, bs, d, B, H, M = c["dtype"], c["bs"], c["d"], c["B"], c["H"], c["M"]
    n_cap = bs * M
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, n_cap + 1, B)]
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, d, generator=g).to(dtype)
    kc = torch.randn(B, H, n_cap, d, generator=g).to(dtype)
    vc = torch.randn(B, H, n_cap, d, generator=g).to(dtype)
    rp, ci = _pattern(c, n_cap, False)
    mask = np.stack(c["masks"]) if c["per_head"] else c["masks"][0]
    dev = torch.device("cuda")
    sl = torch.tensor(lengths, dtype=torch.int32, device=dev)
    what = f"seed {seed}: {c['dtype']} bs{bs} d{d} B{B} H{H} M{M} per_head={c['per_head']}"
    o, lse = bsa.decode(q.to(dev), kc.to(dev), vc.to(dev), sl, rp.to(dev), ci.to(dev), bs,
                        c["scale"], per_head=c["per_head"])
    k8, ks = oracle.quantize_blocks(kc.float().numpy(), bs)
    v8, vs = oracle.quantize_blocks(vc.float().numpy(), bs)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o8, l8 = bsa.decode_int8kv(q.to(dev), t(k8), t(ks), t(v8), t(vs), sl, rp.to(dev),
                               ci.to(dev), bs, c["scale"], per_head=c["per_head"])
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_decode(_f64(q), _f64(kc), _f64(vc), lengths, mask, bs,
                                        c["scale"])
    r8, rl8 = oracle.block_sparse_decode_int8(_f64(q), k8, ks, v8, vs, lengths, mask, bs,
                                              c["scale"])
    _check(_f64(o), ro, dtype, "decode O " + what)
    _check(_f64(lse), rl, dtype, "decode LSE " + what)
    _check(_f64(o8), r8, dtype, "int8 decode O " + what)
    _check(_f64(l8), rl8, dtype, "int8 decode LSE " + what)


@pytest.mark.parametrize("seed", range(300, 340))
def test_forward_row_split_sweep(seed):
    """Random masks with a few dense rows, split with a random chunk size."""
    c = _draw(seed)
    rng = np.random.default_rng(seed)
    dtype, bs, d, B, H = c["dtype"], c["bs"], c["d"], c["B"], c["H"]
    M = int(rng.integers(6, 20))
    N = bs * M
    mask = random_block_mask(M, float(rng.uniform(0.05, 0.4)), seed)
    for r in rng.choice(M, size=int(rng.integers(1, 4)), replace=False):
        mask[r, :] = 1
    causal = c["causal"]
    rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=causal)
    chunk = int(rng.integers(1, 9))
    plan = bsa.plan_row_split(rp, chunk)
    q, k, v = make_qkv(B, H, N, d, dtype, 4000 + seed)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         c["scale"], causal=causal,
                         split=None if plan is None else plan.to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs,
                                                   c["scale"], causal=causal)
    what = f"seed {seed}: {c['dtype']} bs{bs} d{d} B{B} H{H} M{M} causal={causal} " \
           f"chunk={chunk} items={0 if plan is None else plan.n_items}"
    _check(_f64(o), o_ref, dtype, "O " + what)
    _check(_f64(lse), lse_ref, dtype, "LSE " + what)
