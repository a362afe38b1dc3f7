"""Parity of the HIP forward (through the C ABI) with the float64 CPU oracle.

Tolerances (acceptance bar of the method):
  bfloat16 inputs: max |O - O_ref| <= 2e-2 and max |LSE - LSE_ref| <= 2e-2;
  float32 inputs:  ||O - O_ref||_inf / ||O_ref||_inf <= 1e-5, same for LSE.
Small shapes are compared element by element over every output; the full-size
workloads on sampled (batch, head, query block) sets the oracle computes one
by one, plus properties that hold at any size (finite outputs, convex-hull
bound of every row).
"""

import ctypes
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_csr_amd as bsa
import oracle
from workgroup_shapes import refused_cases, runnable_cases
from synthetic_inputs import (WORKLOADS, local_global_block_mask, make_qkv, random_block_mask,
                              workload_block_mask)

pytestmark = pytest.mark.gpu

BF16_ATOL = 2e-2
F32_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa._load()  # fail loudly if the native library is missing


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _mask_for(pattern, N, bs, seed=0):
    M = N // bs
    if pattern == "loglinear":
        return oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs)), None
    if pattern == "ones":
        m = np.ones((M, M), np.uint8)
    elif pattern == "diag":
        m = np.eye(M, dtype=np.uint8)
    elif pattern == "random":
        m = random_block_mask(M, 0.3, seed)
    elif pattern == "local_global":
        m = local_global_block_mask(M)
    elif pattern == "single_col":  # every row sees only block M-1 (not its own)
        m = np.zeros((M, M), np.uint8)
        m[:, M - 1] = 1
    else:
        raise ValueError(pattern)
    return m, m


def _run_gpu(q, k, v, bs, user_mask, scale=None):
    N = q.shape[2]
    rp, ci = bsa.build_pattern(N, bs, mask=user_mask)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs, scale)
    torch.cuda.synchronize()
    return o, lse, rp, ci


def _compare(o, lse, o_ref, lse_ref, dtype, what=""):
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"non-finite output {what}"
    if dtype == torch.float32:
        eo = np.abs(o - o_ref).max() / np.abs(o_ref).max()
        el = np.abs(lse - lse_ref).max() / np.abs(lse_ref).max()
        assert eo <= F32_RTOL and el <= F32_RTOL, f"{what} rel err O {eo:.3e} LSE {el:.3e}"
    else:
        eo = np.abs(o - o_ref).max()
        el = np.abs(lse - lse_ref).max()
        assert eo <= BF16_ATOL and el <= BF16_ATOL, f"{what} abs err O {eo:.3e} LSE {el:.3e}"
    return eo, el


SMALL = []
for dt in ("bf16", "f32"):
    for bs in (32, 64):
        for d in (64, 128):
            for pattern, B, H, M in (("loglinear", 1, 2, 8), ("loglinear", 2, 3, 7),
                                     ("ones", 1, 1, 5), ("diag", 2, 1, 3),
                                     ("random", 3, 2, 9), ("local_global", 1, 2, 12),
                                     ("single_col", 1, 1, 4), ("loglinear", 1, 1, 1)):
                SMALL.append((dt, bs, d, pattern, B, H, M))


@pytest.mark.parametrize("dt,bs,d,pattern,B,H,M", SMALL)
def test_small_full_parity(dt, bs, d, pattern, B, H, M):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    N = bs * M
    seed = zlib.crc32(repr((dt, bs, d, pattern, B, H, M)).encode()) % 1000
    q, k, v = make_qkv(B, H, N, d, dtype, seed)
    mask, user = _mask_for(pattern, N, bs, seed)
    o, lse, _, _ = _run_gpu(q, k, v, bs, user)
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, dtype, f"{dt} bs{bs} d{d} {pattern}")


def test_tiny_workload_full():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, 0)
    o, lse, rp, ci = _run_gpu(q, k, v, w.block_size, None)
    assert int(rp[-1]) == 39
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(w.N, w.block_size))
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, w.block_size)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, torch.float32, "tiny")


def _convex_hull_check(o, v, mask, bs, tol):
    """Every output row lies within [min, max] of the V rows it attends to."""
    M = mask.shape[0]
    for qb in range(M):
        sel = np.repeat(mask[qb] != 0, bs)
        lo = v[sel].min(axis=0) - tol
        hi = v[sel].max(axis=0) + tol
        rows = o[qb * bs:(qb + 1) * bs]
        assert np.all(rows >= lo) and np.all(rows <= hi), f"query block {qb}"


def test_worked_example_full():
    w = WORKLOADS["worked_example"]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, 0)
    o, lse, rp, ci = _run_gpu(q, k, v, w.block_size, None)
    assert int(rp[-1]) == 1251
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(w.N, w.block_size))
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    o_ref, lse_ref = oracle.block_sparse_attention(qf, kf, vf, mask, w.block_size)
    eo, el = _compare(_f64(o), _f64(lse), o_ref, lse_ref, torch.bfloat16, "worked example")
    print(f"worked example: max|dO| {eo:.3e} max|dLSE| {el:.3e}")
    _convex_hull_check(_f64(o)[0, 3], vf[0, 3], mask, w.block_size, 1e-2)


# Sampled (batch, head) pairs spread over the grid's XCD ranges, and query
# blocks that include the dense rows, the anchors, both ends and a stride
# through the rest (None: every block of the head).
_LONG_QB = sorted({0, 1, 2, 3, 255, 256, 257, 509, 510, 511} | set(range(5, 512, 17)))
_LG_QB = sorted({0, 1, 2, 5, 63, 64, 100, 126, 127} | set(range(3, 128, 11)))


@pytest.mark.parametrize("name,heads,qblocks", [
    ("local_global", [(0, 0), (0, 9), (1, 3), (1, 6), (1, 15)], _LG_QB),
    ("random_mask", [(0, 0), (19, 5), (45, 2), (77, 3), (101, 6), (127, 7)], None),
    ("long", [(0, 0), (0, 9), (0, 18), (0, 31)], _LONG_QB),
    ("worked_example_b32", [(0, 0), (9, 4), (17, 2), (24, 1), (31, 7)], None),
])
def test_full_size_workload_sampled(name, heads, qblocks):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, 0)
    user = workload_block_mask(w, seed=0)
    o, lse, rp, ci = _run_gpu(q, k, v, w.block_size, user)
    mask = user if user is not None else oracle.block_mask_from_sets(
        oracle.loglinear_block_sets(w.N, w.block_size))
    assert int(rp[-1]) == int((mask != 0).sum())
    o_all = o.float()
    assert torch.isfinite(o_all).all() and torch.isfinite(lse).all()
    worst = (0.0, 0.0)
    for b, h in heads:
        o_ref, lse_ref = oracle.block_sparse_attention_head(
            _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), mask, w.block_size,
            query_blocks=qblocks)
        rows = np.isfinite(lse_ref)
        eo, el = _compare(_f64(o[b, h])[rows], _f64(lse[b, h])[rows], o_ref[rows],
                          lse_ref[rows], w.torch_dtype, f"{name} b{b} h{h}")
        worst = (max(worst[0], eo), max(worst[1], el))
    print(f"{name}: max|dO| {worst[0]:.3e} max|dLSE| {worst[1]:.3e}")
    b, h = heads[0]
    _convex_hull_check(_f64(o[b, h]), _f64(v[b, h]), mask, w.block_size, 1e-2)


def test_scale_override_and_side_stream():
    q, k, v = make_qkv(2, 2, 64 * 6, 64, torch.bfloat16, 5)
    mask, user = _mask_for("random", 64 * 6, 64, 5)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(64 * 6, 64, mask=user)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), 64,
                             scale=0.3)
    s.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, 64,
                                                   scale=0.3)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, torch.bfloat16, "scale 0.3")


def test_null_lse_through_c_abi():
    q, k, v = make_qkv(1, 2, 256, 64, torch.bfloat16, 9)
    dev = torch.device("cuda")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    rp, ci = bsa.build_pattern(256, 32)
    rp, ci = rp.to(dev), ci.to(dev)
    o_ref, _ = bsa.forward(q, k, v, rp, ci, 32)
    o = torch.empty_like(q)
    lib = bsa._load()
    st = lib.bsa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None, 1, 2, 256,
                         64, 32, 1, rp.data_ptr(), ci.data_ptr(), ci.numel(),
                         ctypes.c_float(0.0), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_deterministic_repeat():
    q, k, v = make_qkv(2, 4, 4096, 64, torch.bfloat16, 3)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(4096, 32)
    args = (q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), 32)
    o1, l1 = bsa.forward(*args)
    o2, l2 = bsa.forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_nan_propagates_only_to_rows_that_see_it():
    bs, M, d = 32, 8, 64
    N = bs * M
    q, k, v = make_qkv(1, 1, N, d, torch.bfloat16, 2)
    k[0, 0, 5 * bs + 3, 7] = float("nan")  # a key in block 5
    o, lse, rp, ci = _run_gpu(q, k, v, bs, None)
    sets = oracle.loglinear_block_sets(N, bs)
    of = _f64(o)[0, 0]
    for qb in range(M):
        rows = of[qb * bs:(qb + 1) * bs]
        if 5 in sets[qb]:
            assert np.isnan(rows).all(), qb
        else:
            assert np.isfinite(rows).all(), qb


@pytest.mark.parametrize("dt,bs,d,group,key_split", runnable_cases())
def test_every_workgroup_shape(dt, bs, d, group, key_split):
    """bsa_forward_ex: every (group, key_split) the library runs computes the
    oracle's result, on a ragged case (M = 11 query blocks is a multiple of no
    group size)."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 3, 11
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, dtype, 17)
    mask = random_block_mask(M, 0.35, 17)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs, mask=mask)
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         group=group, key_split=key_split)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), mask, bs)
    _compare(_f64(o), _f64(lse), o_ref, lse_ref, dtype, f"{dt} bs{bs} d{d} G{group} KS{key_split}")


@pytest.mark.parametrize("dt,bs,d,group,key_split", refused_cases())
def test_refused_workgroup_shapes(dt, bs, d, group, key_split):
    """Shapes that are not instantiated, or whose LDS ring does not fit a
    workgroup, are refused with BSA_ERR_INVALID_ARGUMENT (status 2) before any
    launch; so are shapes of more than 8 waves."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 1, 1, 11
    N = bs * M
    q, k, v = make_qkv(B, H, N, d, dtype, 17)
    dev = torch.device("cuda")
    rp, ci = bsa.build_pattern(N, bs)
    for g, ks in ((group, key_split), (8, 2)):
        with pytest.raises(bsa.BsaError) as e:
            bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                        group=g, key_split=ks)
        assert e.value.status == 2


@pytest.mark.parametrize("dt,bs,d,group,key_split",
                         runnable_cases([("bf16", 32, 64), ("f32", 64, 128), ("bf16", 64, 128)]))
def test_hand_made_csr_empty_rows_and_out_of_range_entries(dt, bs, d, group, key_split):
    """A CSR not from bsa_build_pattern: a row with no entry and a row with
    only entries outside [0, M) get O = 0 and LSE = -inf (no NaN, the failure
    the log-linear page traces to empty rows); entries outside [0, M) inside a
    row are skipped; every other row matches the oracle."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, M = 2, 2, 11
    N = bs * M
    mask = random_block_mask(M, 0.35, 23)
    rows = [sorted(np.nonzero(mask[i])[0].tolist()) for i in range(M)]
    rows[1] = []                       # empty
    rows[4] = [-3, M + 2]              # only entries outside [0, M)
    rows[6] = [-1, 0, 6, M]            # effective {0, 6}
    rp = torch.tensor(np.cumsum([0] + [len(r) for r in rows]), dtype=torch.int32)
    ci = torch.tensor([j for r in rows for j in r], dtype=torch.int32)
    q, k, v = make_qkv(B, H, N, d, dtype, 29)
    dev = torch.device("cuda")
    o, lse = bsa.forward(q.to(dev), k.to(dev), v.to(dev), rp.to(dev), ci.to(dev), bs,
                         group=group, key_split=key_split)
    torch.cuda.synchronize()
    o, lse = _f64(o), _f64(lse)
    eff = np.zeros((M, M), np.uint8)
    for i, r in enumerate(rows):
        for j in r:
            if 0 <= j < M:
                eff[i, j] = 1
    dead = [i for i in range(M) if not eff[i].any()]
    assert dead == [1, 4]
    for i in dead:
        sl = slice(i * bs, (i + 1) * bs)
        assert np.all(o[:, :, sl] == 0) and np.all(lse[:, :, sl] == -np.inf)
        eff[i, i] = 1  # any non-empty row for the oracle; these rows are not compared
    o_ref, lse_ref = oracle.block_sparse_attention(_f64(q), _f64(k), _f64(v), eff, bs)
    live = np.concatenate([np.arange(i * bs, (i + 1) * bs) for i in range(M) if i not in dead])
    _compare(o[:, :, live], lse[:, :, live], o_ref[:, :, live], lse_ref[:, :, live], dtype,
             f"{dt} bs{bs} d{d} G{group} KS{key_split}")


@pytest.mark.parametrize("B,H", [(1, 1), (2, 2)])
def test_longest_supported_blocks_sampled(B, H):
    """N = 131072 at block 32: M = 4096 query blocks, the largest entry list
    and bitmaps the kernel keeps in LDS.  B = H = 1 runs the one-block
    workgroups, B = H = 2 the four-block ones; sampled query blocks (start,
    anchors at M/2 and M-1, end) against the oracle."""
    N, d, bs = 131072, 64, 32
    M = N // bs
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, 3)
    o, lse, rp, ci = _run_gpu(q, k, v, bs, None)
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    assert int(rp[-1]) == int(mask.sum())
    qblocks = [0, 1, 5, M // 2 - 1, M // 2, M // 2 + 3, M - 2, M - 1]
    for b, h in {(0, 0), (B - 1, H - 1)}:
        o_ref, lse_ref = oracle.block_sparse_attention_head(
            _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), mask, bs, query_blocks=qblocks)
        rows = np.isfinite(lse_ref)
        _compare(_f64(o[b, h])[rows], _f64(lse[b, h])[rows], o_ref[rows], lse_ref[rows],
                 torch.bfloat16, f"N={N} b{b} h{h}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
