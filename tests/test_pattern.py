"""bsa_build_pattern (C++ host builder, through the C ABI) against the oracle.

CSR output must be bit-exact: same row_ptr, same col_idx, int32.
"""

import ctypes

import numpy as np
import pytest

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import (WORKLOADS, bernoulli_block_mask, local_global_block_mask,
                              random_block_mask, workload_block_mask)


def _oracle_csr_loglinear(N, bs, **kw):
    return oracle.csr_from_block_mask(oracle.block_mask_from_sets(
        oracle.loglinear_block_sets(N, bs, **kw)))


def _assert_same(got, want):
    row_ptr, col_idx = got
    want_rp, want_ci = want
    assert row_ptr.dtype == col_idx.dtype  # torch.int32
    assert str(row_ptr.dtype) == "torch.int32"
    np.testing.assert_array_equal(row_ptr.numpy(), want_rp)
    np.testing.assert_array_equal(col_idx.numpy(), want_ci)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_patterns_bit_exact(name):
    w = WORKLOADS[name]
    mask = workload_block_mask(w, seed=0)
    if mask is None:
        got = bsa.build_pattern(w.N, w.block_size)
        want = _oracle_csr_loglinear(w.N, w.block_size)
    else:
        got = bsa.build_pattern(w.N, w.block_size, mask=mask)
        want = oracle.csr_from_block_mask(mask)
    _assert_same(got, want)


def test_worked_example_nnz():
    row_ptr, col_idx = bsa.build_pattern(4096, 32)
    assert int(row_ptr[-1]) == col_idx.numel() == 1251
    assert col_idx[:6].tolist() == [0, 1, 2, 4, 64, 127]


def test_local_global_counts():
    rp, _ = bsa.build_pattern(8192, 64, mask=local_global_block_mask(128))
    sizes = np.diff(rp.numpy())
    assert sizes[0] == sizes[-1] == 128
    assert int(rp[-1]) == 1622


@pytest.mark.parametrize("M", [1, 2, 3, 5, 6, 7, 8, 100, 1000])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_loglinear_sweep(M, bs):
    _assert_same(bsa.build_pattern(M * bs, bs), _oracle_csr_loglinear(M * bs, bs))


@pytest.mark.parametrize("radius,k_max,globals_", [(0, None, None), (2, None, None),
                                                   (1, 0, None), (1, 3, None), (1, 40, None),
                                                   (1, None, []), (1, None, [5, 5, 0]),
                                                   (3, 12, [1, 2, 3, 4, 5, 6, 7])])
def test_loglinear_parameters(radius, k_max, globals_):
    N, bs = 300 * 32, 32
    got = bsa.build_pattern(N, bs, local_radius=radius, k_max=k_max, global_blocks=globals_)
    kw = {"local_radius": radius}
    if k_max is not None:
        kw["k_max"] = k_max
    if globals_ is not None:
        kw["global_blocks"] = globals_
    if k_max == 0 and radius == 0 and globals_ == []:
        pytest.skip("empty rows")
    _assert_same(got, _oracle_csr_loglinear(N, bs, **kw))


@pytest.mark.parametrize("seed", range(200))
def test_random_masks(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 70))
    p = float(rng.uniform(0.02, 1.0))
    mask = random_block_mask(M, p, seed)
    # arbitrary nonzero byte values select too
    mask = mask * rng.integers(1, 256, size=mask.shape).astype(np.uint8)
    _assert_same(bsa.build_pattern(M * 64, 64, mask=mask),
                 oracle.csr_from_block_mask(mask))


def test_bernoulli_mask_statistics():
    mask = bernoulli_block_mask(32, seed=0)
    assert np.all(np.diag(mask) == 1)
    rp, ci = bsa.build_pattern(2048, 64, mask=mask)
    assert int(rp[-1]) == int(mask.sum())


def _status(excinfo):
    return excinfo.value.status


def test_error_empty_row():
    mask = np.eye(4, dtype=np.uint8)
    mask[2, 2] = 0
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(4 * 32, 32, mask=mask)
    assert _status(e) == 4


def test_error_global_out_of_range():
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(256, 32, global_blocks=[8])
    assert _status(e) == 5
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(256, 32, global_blocks=[-1])
    assert _status(e) == 5


@pytest.mark.parametrize("N,bs", [(100, 32), (0, 32), (64, 0), (-64, 32)])
def test_error_shape(N, bs):
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(N, bs)
    assert _status(e) == 3


def test_error_buffer_too_small_reports_nnz():
    import ctypes
    lib = bsa._load()
    desc = bsa._desc(4096, 32, None, None, None, None, None, False, None, None, None, None, [])
    nnz = ctypes.c_int64(-1)
    buf = (ctypes.c_int32 * 10)()
    st = lib.bsa_build_pattern(ctypes.byref(desc), None, buf, 10, ctypes.byref(nnz))
    assert st == 6 and nnz.value == 1251
    st = lib.bsa_build_pattern(None, None, None, 0, ctypes.byref(nnz))
    assert st == 1
    st = lib.bsa_build_pattern(ctypes.byref(desc), None, None, 0, None)
    assert st == 1
    desc.kind = 7
    assert lib.bsa_build_pattern(ctypes.byref(desc), None, None, 0, ctypes.byref(nnz)) == 2
    desc.kind = 1  # block mask without a mask pointer
    assert lib.bsa_build_pattern(ctypes.byref(desc), None, None, 0, ctypes.byref(nnz)) == 1


# ----------------------------------------------------------------------------- further kinds


def _sets_from_csr(rp, ci):
    rp, ci = rp.numpy(), ci.numpy()
    return [set(int(j) for j in ci[rp[i]:rp[i + 1]]) for i in range(len(rp) - 1)]


def _check_sorted_unique(rp, ci):
    rp, ci = rp.numpy(), ci.numpy()
    for i in range(len(rp) - 1):
        row = ci[rp[i]:rp[i + 1]]
        assert (np.diff(row) > 0).all()


@pytest.mark.parametrize("M,bs,w,dil,g", [(10, 64, 2, 3, None), (128, 32, 4, 1, [0, 127]),
                                          (64, 64, 3, 5, [32]), (1, 32, 0, 1, None),
                                          (200, 32, 7, 11, [0, 199])])
def test_dilated_matches_oracle(M, bs, w, dil, g):
    rp, ci = bsa.build_pattern(M * bs, bs, kind="dilated", window=w, dilation=dil,
                               global_blocks=g)
    ref = oracle.dilated_block_sets(M * bs, bs, window=w, dilation=dil, global_blocks=g or ())
    assert _sets_from_csr(rp, ci) == ref
    _check_sorted_unique(rp, ci)


@pytest.mark.parametrize("M,bs,r,g,nr,seed", [(32, 64, 1, [0], 3, 0), (128, 32, 1, None, 5, 42),
                                              (8, 32, 1, [0, 7], 100, 7),
                                              (512, 64, 2, [0, 511], 4, 2**63 + 5),
                                              (3, 32, 0, None, 1, 1)])
def test_bigbird_matches_oracle(M, bs, r, g, nr, seed):
    rp, ci = bsa.build_pattern(M * bs, bs, kind="bigbird", local_radius=r, global_blocks=g,
                               num_random=nr, seed=seed)
    ref = oracle.bigbird_block_sets(M * bs, bs, num_random=nr, seed=seed, local_radius=r,
                                    global_blocks=g or ())
    assert _sets_from_csr(rp, ci) == ref
    _check_sorted_unique(rp, ci)


@pytest.mark.parametrize("kind", ["loglinear", "mask", "dilated", "bigbird"])
def test_causal_matches_oracle(kind):
    N, bs = 4096, 32
    M = N // bs
    if kind == "loglinear":
        sets = oracle.loglinear_block_sets(N, bs)
        kw = {}
    elif kind == "mask":
        m = random_block_mask(M, 0.3, 9)
        sets = [set(np.nonzero(m[i])[0].tolist()) for i in range(M)]
        kw = {"mask": m}
    elif kind == "dilated":
        sets = oracle.dilated_block_sets(N, bs, window=3, dilation=2, global_blocks=[0])
        kw = {"window": 3, "dilation": 2, "global_blocks": [0]}
    else:
        sets = oracle.bigbird_block_sets(N, bs, num_random=3, seed=11, global_blocks=[0])
        kw = {"num_random": 3, "seed": 11, "global_blocks": [0]}
    rp, ci = bsa.build_pattern(N, bs, kind=kind, causal=True, **kw)
    assert _sets_from_csr(rp, ci) == oracle.causal_block_sets(sets)


def test_causal_row_losing_every_block_is_an_empty_row():
    m = np.zeros((4, 4), np.uint8)
    m[:, 3] = 1  # every row selects only the last block
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(128, 32, mask=m, causal=True)
    assert e.value.status == 4


@pytest.mark.parametrize("kw,status", [({"kind": "dilated", "window": -1, "dilation": 1}, 2),
                                       ({"kind": "dilated", "window": 1, "dilation": 0}, 2),
                                       ({"kind": "bigbird", "num_random": -1, "seed": 0}, 2),
                                       ({"kind": "dilated", "window": 1, "dilation": 1,
                                         "global_blocks": [128]}, 5),
                                       ({"kind": "bigbird", "num_random": 1, "seed": 0,
                                         "global_blocks": [-1]}, 5)])
def test_new_kinds_reject_bad_input(kw, status):
    with pytest.raises(bsa.BsaError) as e:
        bsa.build_pattern(4096, 32, **kw)
    assert e.value.status == status


def test_seven_anchor_loglinear_matches_oracle():
    M = 128
    anchors = [0, 21, 42, 64, 85, 106, 127]
    rp, ci = bsa.build_pattern(M * 32, 32, global_blocks=anchors)
    assert _sets_from_csr(rp, ci) == oracle.loglinear_block_sets(M * 32, 32, global_blocks=anchors)


def test_stack_head_patterns_offsets():
    a = bsa.build_pattern(1024, 32)
    b = bsa.build_pattern(1024, 32, kind="dilated", window=2, dilation=2)
    rp, ci = bsa.stack_head_patterns([a, b])
    M = 32
    assert rp.numel() == 2 * (M + 1) and ci.numel() == a[1].numel() + b[1].numel()
    assert (rp[:M + 1] == a[0]).all() and (rp[M + 1:] == b[0] + a[1].numel()).all()
    assert (ci[:a[1].numel()] == a[1]).all() and (ci[a[1].numel():] == b[1]).all()


@pytest.mark.parametrize("kind", ["loglinear", "mask", "bigbird"])
def test_transpose_pattern_matches_numpy(kind):
    N, bs = 4096, 32
    M = N // bs
    kw = {"mask": random_block_mask(M, 0.2, 4)} if kind == "mask" else (
        {"kind": "bigbird", "num_random": 3, "seed": 9} if kind == "bigbird" else {})
    rp, ci = bsa.build_pattern(N, bs, **kw)
    cp, ri = bsa.transpose_pattern(rp, ci)
    dense = oracle.block_mask_from_csr(rp.numpy(), ci.numpy(), M)
    cp_ref, ri_ref = oracle.csr_from_block_mask(dense.T.copy())
    assert np.array_equal(cp.numpy(), cp_ref) and np.array_equal(ri.numpy(), ri_ref)


def test_transpose_pattern_errors():
    import torch
    rp = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(bsa.BsaError) as e:
        bsa.transpose_pattern(rp, torch.tensor([0, 2], dtype=torch.int32))
    assert e.value.status == 5
    with pytest.raises(bsa.BsaError) as e:
        bsa.transpose_pattern(torch.tensor([0, 2, 1], dtype=torch.int32),
                              torch.tensor([0, 1], dtype=torch.int32))
    assert e.value.status == 3


def test_pattern_order_long_blocks_first():
    # worked example: the anchors' columns (0, 64, 127) hold all 128 query
    # blocks (13x the mean); every other column keeps ascending order
    rp, ci = bsa.build_pattern(4096, 32)
    cp, ri = bsa.transpose_pattern(rp, ci)
    co = bsa.pattern_order(cp).numpy().tolist()
    assert co == [0, 64, 127] + [j for j in range(128) if j not in (0, 64, 127)]
    # log-linear rows are all within twice the mean: ascending order
    assert bsa.pattern_order(rp).numpy().tolist() == list(range(128))
    # counts 1, 9, 2, 30, 1, 12: mean 55/6, so only the 30 exceeds twice it
    ptr = np.cumsum([0, 1, 9, 2, 30, 1, 12]).astype(np.int32)
    assert bsa.pattern_order(ptr).numpy().tolist() == [3, 0, 1, 2, 4, 5]
    # counts 1, 40, 1, 1, 40, 50, 1, 1 (twice the mean 33.75): longest first,
    # equal counts ascending, then the rest ascending
    ptr = np.cumsum([0, 1, 40, 1, 1, 40, 50, 1, 1]).astype(np.int32)
    assert bsa.pattern_order(ptr).numpy().tolist() == [5, 1, 4, 0, 2, 3, 6, 7]
    # a uniform pattern keeps ascending order
    ptr = np.arange(0, 5 * 7, 5).astype(np.int32)
    assert bsa.pattern_order(ptr).numpy().tolist() == list(range(6))


def test_pattern_order_errors():
    lib = bsa._load()
    p32 = ctypes.POINTER(ctypes.c_int32)
    ptr = np.array([0, 2, 1, 3], np.int32)
    out = np.zeros(3, np.int32)
    assert lib.bsa_pattern_order(3, ptr.ctypes.data_as(p32), out.ctypes.data_as(p32)) == 3
    ptr = np.array([1, 2, 3], np.int32)
    assert lib.bsa_pattern_order(2, ptr.ctypes.data_as(p32), out.ctypes.data_as(p32)) == 3
    assert lib.bsa_pattern_order(0, ptr.ctypes.data_as(p32), out.ctypes.data_as(p32)) == 3
    assert lib.bsa_pattern_order(2, None, out.ctypes.data_as(p32)) == 1


def _plan_raw(ptr, chunk, item_cap=None):
    lib = bsa._load()
    p32 = ctypes.POINTER(ctypes.c_int32)
    ptr = np.ascontiguousarray(ptr, dtype=np.int32)
    M = ptr.size - 1
    cap = int(ptr[-1]) if item_cap is None else item_cap
    heavy = np.full(M, 7, np.uint8)
    items = np.zeros(3 * max(cap, 1), np.int32)
    rows = np.zeros(3 * M, np.int32)
    n_items, n_rows = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib.bsa_plan_row_split(M, ptr.ctypes.data_as(p32), chunk,
                                heavy.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                items.ctypes.data_as(p32), cap, ctypes.byref(n_items),
                                rows.ctypes.data_as(p32), ctypes.byref(n_rows))
    return st, heavy, items[:3 * max(n_items.value, 0)].reshape(-1, 3), \
        rows[:3 * max(n_rows.value, 0)].reshape(-1, 3), n_items.value


def test_row_split_plan_local_global():
    # local+global at M = 128: rows 0 and M - 1 hold all 128 blocks, the rest
    # 7..11 (mean 12.67 -> default chunk 16): two heavy rows of 8 items each
    M = 128
    rp, ci = bsa.build_pattern(64 * M, 64, mask=local_global_block_mask(M))
    plan = bsa.plan_row_split(rp)
    assert plan.heavy.numpy().nonzero()[0].tolist() == [0, M - 1]
    assert plan.rows.tolist() == [[0, 0, 8], [M - 1, 8, 8]]
    r = rp.numpy()
    want = [[0, r[0] + 16 * i, r[0] + 16 * (i + 1)] for i in range(8)]
    want += [[M - 1, r[M - 1] + 16 * i, r[M - 1] + 16 * (i + 1)] for i in range(8)]
    assert plan.items.tolist() == want
    # every entry of a heavy row lies in exactly one of its items
    for row, first, count in plan.rows.tolist():
        its = plan.items[first:first + count].numpy()
        assert its[0, 1] == r[row] and its[-1, 2] == r[row + 1]
        assert (its[1:, 1] == its[:-1, 2]).all()
    # the log-linear pattern has no heavy row
    assert bsa.plan_row_split(bsa.build_pattern(4096, 32)[0]) is None


def test_row_split_plan_boundaries_and_errors():
    # counts 20, 21, 3 with chunk 10: 20 = 2 chunk is not heavy, 21 is (3 items)
    ptr = np.cumsum([0, 20, 21, 3])
    st, heavy, items, rows, n = _plan_raw(ptr, 10)
    assert st == 0 and heavy.tolist() == [0, 1, 0] and n == 3
    assert items.tolist() == [[1, 20, 30], [1, 30, 40], [1, 40, 41]]
    assert rows.tolist() == [[1, 0, 3]]
    # default chunk: mean 44/3 -> 15 -> 16; nothing exceeds 32
    st, heavy, items, rows, n = _plan_raw(ptr, 0)
    assert st == 0 and heavy.tolist() == [0, 0, 0] and n == 0
    # too few item slots: the count is still reported
    st, _, _, _, n = _plan_raw(ptr, 10, item_cap=2)
    assert st == 6 and n == 3
    lib = bsa._load()
    p32 = ctypes.POINTER(ctypes.c_int32)
    bad = np.array([0, 5, 3], np.int32)
    out8 = np.zeros(2, np.uint8)
    buf = np.zeros(6, np.int32)
    cnt = ctypes.c_int32(0)
    args = lambda ptr_: (2, ptr_.ctypes.data_as(p32), 1,
                         out8.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                         buf.ctypes.data_as(p32), 2, ctypes.byref(cnt), buf.ctypes.data_as(p32),
                         ctypes.byref(cnt))
    assert lib.bsa_plan_row_split(*args(bad)) == 3
    a = list(args(np.array([0, 1, 2], np.int32)))
    a[3] = None
    assert lib.bsa_plan_row_split(*a) == 1


def test_row_split_workspace_bytes():
    lib = bsa._load()
    # one float32 partial per (batch, head, item, 32-row wave): d = 128 holds
    # 4 x 16 registers x 64 lanes + m and l per lane
    per_wave = (4 * 16 * 64 + 2 * 64) * 4
    assert lib.bsa_row_split_workspace_bytes(2, 16, 64, 128, 16) == 2 * 16 * 16 * 2 * per_wave
    assert lib.bsa_row_split_workspace_bytes(1, 1, 32, 64, 3) == 3 * (2 * 16 * 64 + 2 * 64) * 4
    assert lib.bsa_row_split_workspace_bytes(1, 1, 48, 64, 3) == -1
