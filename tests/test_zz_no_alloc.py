"""bsa_backward_noalloc (through the C ABI): the backward with D in the
library's static device scratch instead of a caller workspace.  Its
gradients must equal bsa_backward's bit for bit (same kernels, no atomics),
on two calls in a row, the second with a smaller input; a size beyond the
scratch is refused before any launch; torch allocates nothing during the
call."""

import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
from synthetic_inputs import local_global_block_mask, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _case(dev, B, H, N, d, bs, mask, causal, seed):
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, torch.bfloat16, seed))
    g = make_qkv(B, H, N, d, torch.bfloat16, seed + 1)[0].to(dev)
    rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=causal)
    cp, ri = bsa.transpose_pattern(rp, ci)
    orders = [bsa.pattern_order(t).to(dev) for t in (rp, cp)]
    pat = [t.to(dev) for t in (rp, ci, cp, ri)]
    o, lse = bsa.forward(q, k, v, pat[0], pat[1], bs, causal=causal)
    return q, k, v, o, lse, g, pat, orders


def test_noalloc_backward_matches_backward_twice(dev):
    cases = [  # the second call is smaller than the first
        dict(B=2, H=4, N=2048, d=64, bs=32, mask=None, causal=False, seed=11),
        dict(B=1, H=2, N=1024, d=128, bs=64, mask=local_global_block_mask(16), causal=True,
             seed=12),
    ]
    for c in cases:
        q, k, v, o, lse, g, pat, orders = _case(dev, **c)
        print(f"noalloc case {c['B']}x{c['H']}x{c['N']} d{c['d']} bs{c['bs']}", flush=True)
        ref = bsa.backward(q, k, v, o, lse, g, *pat, c["bs"], causal=c["causal"],
                           row_order=orders[0], col_order=orders[1])
        out = [torch.full_like(q, float("nan")) for _ in range(3)]
        torch.cuda.synchronize()
        allocs = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
        got = bsa.backward_noalloc(q, k, v, o, lse, g, *pat, c["bs"], *out, causal=c["causal"],
                                   row_order=orders[0], col_order=orders[1])
        # torch's allocator was not asked for memory during the call
        assert torch.cuda.memory_stats(dev)["allocation.all.allocated"] == allocs
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), name


def test_noalloc_backward_rejects_sizes_beyond_the_scratch():
    lib = bsa._load()
    rows = int(lib.bsa_backward_noalloc_max_rows())
    assert rows == 1 << 22
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: refused before any HIP call
    B, H, N = 2, 8, (rows // 16) + 64  # B * H * N > rows
    st = lib.bsa_backward_noalloc(*([fake] * 9), B, H, N, 64, 32, 1, *([fake] * 4), None, None,
                                  int(N // 32), 0.0, 0, None)
    assert st == 6  # BSA_ERR_BUFFER_TOO_SMALL
