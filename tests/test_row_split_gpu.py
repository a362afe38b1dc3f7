"""Rows split across workgroups (bsa_forward_split through the C ABI):
parity with the float64 oracle when the long rows of a pattern -- the global
rows of a banded local+global mask -- are cut into items, computed as partial
states on separate workgroups and merged.  Small chunk sizes split nearly
every row, so the merge meets many items per row, rows whose items see no
key (causal), and rows of a single item."""

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import WORKLOADS, local_global_block_mask, make_qkv, random_block_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _compare(o, lse, o_ref, lse_ref, dtype, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), what
    if dtype == torch.bfloat16:
        assert np.abs(o - o_ref).max() <= 2e-2, what
        assert np.abs(lse - lse_ref).max() <= 2e-2, what
    else:
        assert np.abs(o - o_ref).max() <= 1e-5 * np.abs(o_ref).max(), what
        assert np.abs(lse - lse_ref).max() <= 1e-5 * np.abs(lse_ref).max(), what


@pytest.mark.parametrize("chunk", [1, 4, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt,bs,d", [("bf16", 32, 64), ("bf16", 64, 128), ("f32", 32, 128),
                                     ("f32", 64, 64)])
def test_split_rows_parity(dt, bs, d, causal, chunk):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 2, 16
    N = bs * M
    mask = local_global_block_mask(M)
    q, k, v = make_qkv(B, H, N, d, dtype, 71)
    rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=causal)
    plan = bsa.plan_row_split(rp, chunk)
    if chunk == 0:  # the default chunk (16 here) leaves rows of 16 entries whole
        assert plan is None
        plan = bsa.plan_row_split(rp, 5)
    assert plan is not None and plan.n_rows >= 1  # causal: only the last row stays long
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         causal=causal, split=plan.to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs,
                                                   causal=causal)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, dtype,
             f"{dt} bs{bs} d{d} causal={causal} chunk={chunk} items={plan.n_items}")


def test_split_matches_plain_forward_on_the_other_rows():
    # the rows the plan leaves whole come from the same kernel as without it
    bs, d, M = 64, 128, 24
    N = bs * M
    mask = random_block_mask(M, 0.3, 5)
    mask[3, :] = 1
    mask[17, :] = 1
    q, k, v = (t.cuda() for t in make_qkv(2, 3, N, d, torch.bfloat16, 72))
    rp, ci = bsa.build_pattern(N, bs, mask=mask)
    plan = bsa.plan_row_split(rp, 6)
    heavy = plan.heavy.numpy().astype(bool)
    assert heavy[3] and heavy[17]
    o1, l1 = bsa.forward(q, k, v, rp.cuda(), ci.cuda(), bs, split=plan.to("cuda"))
    o0, l0 = bsa.forward(q, k, v, rp.cuda(), ci.cuda(), bs)
    torch.cuda.synchronize()
    light = np.repeat(~heavy, bs)
    assert torch.equal(o1[:, :, light], o0[:, :, light])
    assert torch.equal(l1[:, :, light], l0[:, :, light])
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs)
    _compare(_f64(o1), _f64(l1), o_ref, lse_ref, torch.bfloat16, "random mask, two dense rows")


def test_split_local_global_workload_sampled():
    """The local+global workload at full size (B=2 H=16 N=8192 d=128 block
    64): its two global rows per head split into 8 items each; the heavy rows
    and a few others checked against the oracle on sampled heads."""
    w = WORKLOADS["local_global"]
    M = w.N // w.block_size
    mask = local_global_block_mask(M)
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, 0)
    rp, ci = bsa.build_pattern(w.N, w.block_size, mask=mask)
    plan = bsa.plan_row_split(rp)
    assert plan.rows.tolist() == [[0, 0, 8], [M - 1, 8, 8]]
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), w.block_size,
                         split=plan.to(dev))
    torch.cuda.synchronize()
    blocks = [0, 1, 64, M - 2, M - 1]
    ref_o, ref_l = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, w.block_size,
                                                 heads=[(0, 0), (1, 15), (1, 7)],
                                                 query_blocks=blocks)
    for b, h in [(0, 0), (1, 15), (1, 7)]:
        for qb in blocks:
            sl = slice(qb * w.block_size, (qb + 1) * w.block_size)
            assert np.abs(_f64(o[b, h, sl]) - ref_o[b, h, sl]).max() <= 2e-2
            assert np.abs(_f64(lse[b, h, sl]) - ref_l[b, h, sl]).max() <= 2e-2


def test_split_forward_in_a_graph_replays():
    """Captured in a HIP graph (all three launches), replayed three times with
    new inputs and eager work in between: every replay equals the eager call
    on the same inputs."""
    bs, d, M = 64, 128, 32
    N = bs * M
    mask = local_global_block_mask(M)
    rp, ci = bsa.build_pattern(N, bs, mask=mask)
    plan = bsa.plan_row_split(rp, 8)
    assert plan is not None
    dev = torch.device("cuda")
    rp, ci, plan = rp.to(dev), ci.to(dev), plan.to(dev)
    q, k, v = (t.to(dev) for t in make_qkv(2, 4, N, d, torch.bfloat16, 81))
    need = bsa._load().bsa_row_split_workspace_bytes(2, 4, bs, d, plan.n_items)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    run = lambda: bsa.forward(q, k, v, rp, ci, bs, out=o, lse=lse, split=plan, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        nq, nk, nv = (t.to(dev) for t in make_qkv(2, 4, N, d, torch.bfloat16, 90 + rep))
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        og, lg = o.clone(), lse.clone()
        eo, el = bsa.forward(q, k, v, rp, ci, bs, split=plan)  # eager, own outputs
        torch.cuda.synchronize()
        assert torch.equal(og, eo) and torch.equal(lg, el), f"replay {rep}"


@pytest.mark.parametrize("chunk", [12, 5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt,bs,d", [("bf16", 32, 64), ("bf16", 64, 128), ("f32", 64, 64)])
def test_split_items_beside_the_groups(dt, bs, d, causal, chunk):
    """A grid of 8192 query blocks (B=8, H=32, M=32): several query blocks per
    workgroup, so the heavy rows' items run in the same launch as the groups,
    G items per workgroup (item t + g * tuples as block g), and the merge
    follows.  Chunk 12 gives 3 items per dense row (6 in all: a workgroup
    whose last block has no item at G = 4); chunk 5 splits ordinary rows
    too.  Sampled heads against the oracle on every row."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 8, 32, 32
    N = bs * M
    mask = local_global_block_mask(M)
    q, k, v = make_qkv(B, H, N, d, dtype, 83)
    rp, ci = bsa.build_pattern(N, bs, mask=mask, causal=causal)
    plan = bsa.plan_row_split(rp, chunk)
    assert plan is not None
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         causal=causal, split=plan.to(dev))
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 17), (7, 31)):
        f = lambda x: _f64(x[b:b + 1, h:h + 1])
        o_ref, lse_ref = oracle.block_sparse_attention(f(q), f(k), f(v), mask, bs,
                                                       causal=causal)
        _compare(f(o), _f64(lse[b:b + 1, h:h + 1]), o_ref, lse_ref, dtype,
                 f"{dt} bs{bs} d{d} causal={causal} chunk={chunk} ({b}, {h})")
