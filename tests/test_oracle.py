"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: the pattern is checked against
hand-derived rows of the pages' worked examples and a closed-form offset
description; the attention against library routines (torch's
scaled_dot_product_attention in float64, scipy's logsumexp), a textbook loop,
closed forms and invariants.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import (block_mask_from_csr, block_mask_from_sets, block_sparse_attention,
                    block_sparse_attention_head, ceil_log2, csr_from_block_mask,
                    local_global_token_mask, loglinear_block_sets, token_mask_to_block_mask)
from synthetic_inputs import local_global_block_mask, random_block_mask


# ----------------------------------------------------------------------------- pattern


def _check_golden_loglinear(g, sets):
    N = int(g["N"][0])
    bs = int(g["block_size"][0])
    M = int(g["M"][0])
    assert N // bs == M == len(sets)
    assert ceil_log2(M) == int(g["k_max"][0])
    globals_ = [int(x) for x in g["globals"]]
    assert globals_ == [0, M // 2, M - 1]
    for i, cols in g["rows"].items():
        assert sorted(sets[i]) == cols, f"row {i}"
    assert sum(len(s) for s in sets) == int(g["nnz"][0])


def test_pattern_tiny_hand_derived(golden):
    g = golden("tiny_loglinear.txt")
    sets = loglinear_block_sets(int(g["N"][0]), int(g["block_size"][0]))
    _check_golden_loglinear(g, sets)
    assert len(g["rows"]) == len(sets)  # every row is listed


def test_pattern_worked_example_hand_derived(golden):
    g = golden("worked_example_loglinear.txt")
    sets = loglinear_block_sets(4096, 32)
    _check_golden_loglinear(g, sets)
    strides = [(2 ** k) // 32 for k in range(1, ceil_log2(128) + 1)]
    assert strides == [int(x) for x in g["strides"]]
    hist = {}
    for s in sets:
        hist[len(s)] = hist.get(len(s), 0) + 1
    want = dict(tuple(int(x) for x in item.split(":")) for item in g["histogram"])
    assert hist == want


def _closed_form_sets(M, bs):
    """Log-linear rows written as an offset set: {0, +-1} and +-2^e for every
    power of two 2^e * bs <= 2^ceil(log2 M) (the non-zero block strides),
    plus the globals {0, M/2, M-1}.  Block size a power of two."""
    K = (M - 1).bit_length()
    b = bs.bit_length() - 1
    offsets = {0, 1, -1}
    for e in range(0, K - b + 1):
        offsets |= {2 ** e, -(2 ** e)}
    out = []
    for i in range(M):
        s = {i + o for o in offsets if 0 <= i + o < M}
        s |= {0, M // 2, M - 1}
        out.append(s)
    return out


@pytest.mark.parametrize("M,bs", [(1, 32), (2, 32), (3, 32), (4, 16), (5, 32), (7, 64),
                                  (8, 32), (100, 32), (128, 32), (256, 16), (512, 64),
                                  (1000, 32), (2048, 128)])
def test_pattern_closed_form(M, bs):
    sets = loglinear_block_sets(M * bs, bs)
    assert sets == _closed_form_sets(M, bs)


def test_pattern_long_config_counts():
    # N=32768, block 64: strides floor(2^k/64), k=1..9 = 0,0,0,0,0,1,2,4,8.
    sets = loglinear_block_sets(32768, 64)
    assert [(2 ** k) // 64 for k in range(1, 10)] == [0, 0, 0, 0, 0, 1, 2, 4, 8]
    hist = {}
    for s in sets:
        hist[len(s)] = hist.get(len(s), 0) + 1
    # interior rows: offsets {0,+-1,+-2,+-4,+-8} (9) + 3 globals = 12
    assert max(hist) == 12
    assert sum(len(s) for s in sets) == sum(k * v for k, v in hist.items())
    assert sets[300] == {0, 256, 511} | {300 + o for o in (0, 1, -1, 2, -2, 4, -4, 8, -8)}


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_pattern_row_bound_is_logarithmic(bs):
    # |S(i)| <= 3 local + 2 per distinct non-zero stride beyond the local one + 3 globals,
    # i.e. 6 + 2*(ceil(log2 M) - log2 bs), reached for large M: O(log M).
    b = bs.bit_length() - 1
    for p in range(0, 14):
        M = 2 ** p
        sets = loglinear_block_sets(M * bs, bs)
        bound = 6 + 2 * max(0, ceil_log2(M) - b)
        assert max(len(s) for s in sets) <= bound
        if M >= 8:  # row M/4 keeps every offset in range and off the globals
            assert max(len(s) for s in sets) == bound


@pytest.mark.parametrize("M,bs", [(8, 32), (128, 32), (512, 64), (77, 32)])
def test_pattern_own_block_and_symmetry(M, bs):
    sets = loglinear_block_sets(M * bs, bs)
    G = {0, M // 2, M - 1}
    for i, s in enumerate(sets):
        assert i in s  # every token attends to its own block
        for j in s - G:
            if i not in G:
                assert i in sets[j], (i, j)  # local and stride parts are symmetric


def test_pattern_rejects_bad_input():
    with pytest.raises(ValueError):
        loglinear_block_sets(100, 32)
    with pytest.raises(ValueError):
        loglinear_block_sets(256, 32, global_blocks=[8])


@pytest.mark.parametrize("seed", range(5))
def test_csr_roundtrip(seed):
    M = 1 + seed * 13
    mask = random_block_mask(M, 0.3, seed)
    row_ptr, col_idx = csr_from_block_mask(mask)
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr[0] == 0 and row_ptr[-1] == int(mask.astype(bool).sum()) == len(col_idx)
    for i in range(M):
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(np.diff(cols) > 0)  # ascending, unique
    assert np.array_equal(block_mask_from_csr(row_ptr, col_idx, M), mask)


def test_csr_worked_example_row_ptr():
    mask = block_mask_from_sets(loglinear_block_sets(4096, 32))
    row_ptr, col_idx = csr_from_block_mask(mask)
    assert len(row_ptr) == 129 and row_ptr[-1] == 1251
    assert list(col_idx[:6]) == [0, 1, 2, 4, 64, 127]
    assert 1 - 1251 / (128 * 128) == pytest.approx(0.92365, abs=1e-5)


def test_local_global_token_to_block(golden):
    g = golden("local_global_window.txt")
    bs, window = int(g["block_size"][0]), int(g["local_window"][0])
    N = 16 * bs
    tm = local_global_token_mask(N, window, [])
    # coverage of each block distance, counted from the token mask
    cov = {t: int(tm[0:bs, t * bs:(t + 1) * bs].sum()) for t in range(6)}
    want = dict(tuple(int(x) for x in item.split(":")) for item in g["coverage"])
    assert cov == want
    bm = token_mask_to_block_mask(tm, bs)
    r = int(g["band_radius"][0])
    i = np.arange(16)[:, None]
    j = np.arange(16)[None, :]
    assert np.array_equal(bm, (np.abs(i - j) <= r).astype(np.uint8))
    # global tokens [0, -1] do not survive the >50% rule on their own
    bm_g = token_mask_to_block_mask(local_global_token_mask(N, window, [0, -1]), bs)
    assert np.array_equal(bm_g, bm)
    # the workload's block-level reading: the band plus global block rows/columns
    lg = local_global_block_mask(16, radius=r)
    assert np.array_equal(lg[1:-1, 1:-1], bm[1:-1, 1:-1])
    assert lg[0].all() and lg[-1].all() and lg[:, 0].all() and lg[:, -1].all()


def test_token_to_block_partial_last_block():
    # N = 100 at block 64: the last block holds 36 tokens, so its diagonal tile
    # covers 36 * 36 = 1296 real pairs.  A band of half-width w sets
    # 36 + 2 * sum_{t=1..w} (36 - t) of them: 646 at w = 10 (2 * 646 < 1296,
    # dropped) and 696 at w = 11 (kept).  The first diagonal tile sets
    # 64 + 2 * sum_{t=1..w} (64 - t) = 1340 of 4096 at w = 11 (dropped), and
    # the off-diagonal tiles at most 66 of 2304.
    tm10 = local_global_token_mask(100, 10, [])
    tm11 = local_global_token_mask(100, 11, [])
    assert int(tm11[64:, 64:].sum()) == 696 and int(tm10[64:, 64:].sum()) == 646
    assert int(tm11[:64, :64].sum()) == 1340 and int(tm11[:64, 64:].sum()) == 66
    assert np.array_equal(token_mask_to_block_mask(tm10, 64), np.zeros((2, 2), np.uint8))
    assert np.array_equal(token_mask_to_block_mask(tm11, 64), np.array([[0, 0], [0, 1]], np.uint8))
    # a global token sets its whole row and column, negative indices from the end
    g = local_global_token_mask(100, 0, [0, -1])
    assert g[0].all() and g[:, 0].all() and g[99].all() and g[:, 99].all()
    assert int(g.sum()) == 100 + 4 * 98 + 2


# ----------------------------------------------------------------------------- attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, scale=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64)
    m = None if mask is None else torch.from_numpy(mask.astype(bool))
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m,
                                                           scale=scale)
    return out.numpy()


def test_attention_all_ones_equals_dense_sdpa():
    N, d, bs = 256, 64, 32
    q, k, v = (_rand((N, d), s) for s in (1, 2, 3))
    o, lse = block_sparse_attention_head(q, k, v, np.ones((N // bs, N // bs)), bs)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)
    s = q @ k.T / math.sqrt(d)
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_attention_all_ones_textbook_loop():
    N, d, bs = 48, 8, 16
    q, k, v = (_rand((N, d), s) for s in (4, 5, 6))
    o, lse = block_sparse_attention_head(q, k, v, np.ones((3, 3)), bs)
    for r in range(N):
        scores = [sum(q[r, c] * k[j, c] for c in range(d)) / math.sqrt(d) for j in range(N)]
        mx = max(scores)
        e = [math.exp(x - mx) for x in scores]
        z = sum(e)
        for c in range(d):
            assert abs(o[r, c] - sum(e[j] * v[j, c] for j in range(N)) / z) < 1e-12
        assert abs(lse[r] - (mx + math.log(z))) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_attention_block_mask_equals_masked_sdpa(seed):
    bs, M, d = 16, 9, 32
    N = bs * M
    q, k, v = (_rand((N, d), 10 * seed + s) for s in range(3))
    mask = random_block_mask(M, 0.35, seed)
    o, lse = block_sparse_attention_head(q, k, v, mask, bs, scale=0.37)
    token_mask = np.kron(mask, np.ones((bs, bs), dtype=np.uint8))
    np.testing.assert_allclose(o, _sdpa(q, k, v, token_mask, scale=0.37), rtol=0, atol=1e-12)
    s = q @ k.T * 0.37
    s[token_mask == 0] = -np.inf
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_attention_diagonal_mask_is_per_block_dense():
    bs, M, d = 32, 4, 64
    N = bs * M
    q, k, v = (_rand((N, d), s) for s in (7, 8, 9))
    o, _ = block_sparse_attention_head(q, k, v, np.eye(M), bs)
    for b in range(M):
        r = slice(b * bs, (b + 1) * bs)
        np.testing.assert_allclose(o[r], _sdpa(q[r], k[r], v[r]), rtol=0, atol=1e-12)


def test_attention_zero_query_uniform_weights():
    # Q = 0: every selected key gets the same weight, so O is the mean of the
    # selected V rows and LSE = ln(bs * |S(qb)|).  Worked example pattern.
    N, bs, d = 4096, 32, 64
    M = N // bs
    sets = loglinear_block_sets(N, bs)
    mask = block_mask_from_sets(sets)
    q = np.zeros((N, d))
    k = _rand((N, d), 11)
    v = _rand((N, d), 12)
    qbs = [0, 1, 64, 126, 127]
    o, lse = block_sparse_attention_head(q, k, v, mask, bs, query_blocks=qbs)
    assert lse[0] == pytest.approx(math.log(192), abs=1e-12)        # |S(0)| = 6
    assert lse[64 * bs] == pytest.approx(math.log(288), abs=1e-12)  # |S(64)| = 9
    for qb in qbs:
        rows = np.concatenate([np.arange(j * bs, (j + 1) * bs) for j in sorted(sets[qb])])
        want = v[rows].mean(axis=0)
        r = slice(qb * bs, (qb + 1) * bs)
        np.testing.assert_allclose(o[r], np.broadcast_to(want, (bs, d)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[r], math.log(bs * len(sets[qb])), rtol=0, atol=1e-12)


def test_attention_constant_v():
    bs, M, d = 32, 8, 64
    N = bs * M
    q, k = _rand((N, d), 13), _rand((N, d), 14)
    v = np.full((N, d), -1.75)
    mask = block_mask_from_sets(loglinear_block_sets(N, bs))
    o, _ = block_sparse_attention_head(q, k, v, mask, bs)
    np.testing.assert_allclose(o, -1.75, rtol=0, atol=1e-13)


def test_attention_convex_combination_and_normalisation():
    bs, M, d = 32, 16, 64
    N = bs * M
    q, k, v = (3 * _rand((N, d), s) for s in (15, 16, 17))
    mask = block_mask_from_sets(loglinear_block_sets(N, bs))
    o, _, w = block_sparse_attention_head(q, k, v, mask, bs, return_weights=True)
    for qb in range(M):
        token_sel = np.repeat(mask[qb] != 0, bs)
        W = w[qb]
        assert np.all(W >= 0)
        assert np.all(W[:, ~token_sel] == 0)          # unconnected positions hold 0
        np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        r = slice(qb * bs, (qb + 1) * bs)
        lo = v[token_sel].min(axis=0)
        hi = v[token_sel].max(axis=0)
        assert np.all(o[r] >= lo - 1e-12) and np.all(o[r] <= hi + 1e-12)


def test_attention_batched_wrapper_and_sampling():
    B, H, N, d, bs = 2, 3, 128, 16, 32
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    mask = random_block_mask(N // bs, 0.5, 1)
    o, lse = block_sparse_attention(q, k, v, mask, bs, heads=[(1, 2)])
    assert np.isnan(o[0, 0]).all() and np.isfinite(o[1, 2]).all()
    o12, lse12 = block_sparse_attention_head(q[1, 2], k[1, 2], v[1, 2], mask, bs)
    np.testing.assert_array_equal(o[1, 2], o12)
    np.testing.assert_array_equal(lse[1, 2], lse12)


def test_attention_rejects_empty_row():
    with pytest.raises(ValueError):
        block_sparse_attention_head(np.zeros((64, 8)), np.zeros((64, 8)), np.zeros((64, 8)),
                                    np.array([[1, 0], [0, 0]]), 32)


def test_oracle_imports_nothing_from_the_library():
    import os
    import re
    root = os.path.dirname(oracle.__file__)
    for name in os.listdir(root):
        if name.endswith(".py"):
            src = open(os.path.join(root, name)).read()
            assert not re.search(r"block_sparse_attention_csr_amd|synthetic_inputs", src), name


# ----------------------------------------------------------------------------- further rules


def test_splitmix64_published_outputs():
    # First three outputs of the SplitMix64 reference generator started at 0.
    assert [oracle.splitmix64_at(0, n) for n in (1, 2, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


@pytest.mark.parametrize("M,w", [(1, 0), (7, 1), (16, 3), (33, 5)])
def test_dilated_dilation_one_is_a_band(M, w):
    sets = oracle.dilated_block_sets(M * 32, 32, window=w, dilation=1)
    for i, s in enumerate(sets):
        assert s == {j for j in range(M) if abs(i - j) <= w}


def test_dilated_hand_derived():
    # M = 10, window 2, dilation 3: i + 3t for t = -2..2, kept inside [0, 10).
    sets = oracle.dilated_block_sets(640, 64, window=2, dilation=3)
    assert sets[0] == {0, 3, 6}
    assert sets[4] == {1, 4, 7}
    assert sets[9] == {3, 6, 9}
    with_g = oracle.dilated_block_sets(640, 64, window=1, dilation=4, global_blocks=[0, 9])
    assert with_g[5] == {0, 1, 5, 9}
    with pytest.raises(ValueError):
        oracle.dilated_block_sets(640, 64, window=-1, dilation=1)
    with pytest.raises(ValueError):
        oracle.dilated_block_sets(640, 64, window=1, dilation=0)


@pytest.mark.parametrize("M,r,g,nr", [(32, 1, [0], 3), (16, 0, [], 5), (8, 1, [0, 7], 100),
                                      (64, 2, [0, 63], 0)])
def test_bigbird_row_contents(M, r, g, nr):
    sets = oracle.bigbird_block_sets(M * 64, 64, num_random=nr, seed=12345, local_radius=r,
                                     global_blocks=g)
    for i, s in enumerate(sets):
        base = {j for j in range(i - r, i + r + 1) if 0 <= j < M} | set(g)
        assert base <= s
        assert len(s) == len(base) + min(nr, M - len(base))
        assert all(0 <= j < M for j in s)


def test_bigbird_seed_dependence_and_uniform_draw():
    M = 64
    a = oracle.bigbird_block_sets(M * 32, 32, num_random=3, seed=1, local_radius=0)
    b = oracle.bigbird_block_sets(M * 32, 32, num_random=3, seed=1, local_radius=0)
    c = oracle.bigbird_block_sets(M * 32, 32, num_random=3, seed=2, local_radius=0)
    assert a == b and a != c
    # Random picks over many rows spread over all offsets i - j (mod M).
    big = oracle.bigbird_block_sets(512 * 32, 32, num_random=8, seed=7, local_radius=0)
    counts = np.zeros(512)
    for i, s in enumerate(big):
        for j in s - {i}:
            counts[(j - i) % 512] += 1
    expected = counts.sum() / 511
    chi2 = ((counts[1:] - expected) ** 2 / expected).sum()
    assert chi2 < 511 + 6 * math.sqrt(2 * 511)  # 511 degrees of freedom, 6 sigma


def test_causal_block_sets_is_the_lower_triangle():
    sets = loglinear_block_sets(4096, 32)
    causal = oracle.causal_block_sets(sets)
    full = block_mask_from_sets(sets)
    assert (block_mask_from_sets(causal) == np.tril(full)).all()
    assert all(i in s for i, s in enumerate(causal))


# ----------------------------------------------------------------------------- causal / per head


def _causal_textbook(q, k, v, scale):
    N = q.shape[0]
    out = np.zeros_like(q)
    lse = np.zeros(N)
    for r in range(N):
        s = np.array([scale * float(np.dot(q[r], k[j])) for j in range(r + 1)])
        m = s.max()
        p = np.exp(s - m)
        out[r] = (p[:, None] * v[: r + 1]).sum(axis=0) / p.sum()
        lse[r] = m + math.log(p.sum())
    return out, lse


def test_causal_all_ones_equals_causal_sdpa_and_textbook():
    rng = np.random.default_rng(3)
    N, d, bs = 96, 16, 32
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = block_sparse_attention_head(q, k, v, np.ones((3, 3)), bs, causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (q, k, v)), is_causal=True)[0, 0].numpy()
    assert np.abs(o - ref).max() < 1e-12
    o2, lse2 = _causal_textbook(q, k, v, 1 / math.sqrt(d))
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - lse2).max() < 1e-12


def test_causal_zero_query_uniform_over_visible_keys():
    rng = np.random.default_rng(4)
    N, d, bs = 128, 8, 32
    mask = np.array([[1, 0, 0, 0], [1, 1, 0, 0], [0, 1, 1, 0], [1, 0, 1, 1]], np.uint8)
    v = rng.standard_normal((N, d))
    o, lse = block_sparse_attention_head(np.zeros((N, d)), rng.standard_normal((N, d)), v, mask,
                                         bs, causal=True)
    for r in range(N):
        qb = r // bs
        keys = [j for j in range(N) if mask[qb, j // bs] and j <= r]
        assert abs(lse[r] - math.log(len(keys))) < 1e-12
        assert np.abs(o[r] - v[keys].mean(axis=0)).max() < 1e-12


def test_causal_row_without_visible_keys():
    # Query block 0 selects only block 1: with causal masking nothing is left.
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((64, 8)) for _ in range(3))
    o, lse = block_sparse_attention_head(q, k, v, np.array([[0, 1], [1, 1]]), 32, causal=True)
    assert (o[:32] == 0).all() and np.isneginf(lse[:32]).all()
    assert np.isfinite(o[32:]).all() and np.isfinite(lse[32:]).all()


def test_per_head_masks_equal_separate_calls():
    rng = np.random.default_rng(6)
    B, H, N, d, bs = 2, 3, 128, 8, 32
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    masks = np.stack([random_block_mask(4, 0.5, s) for s in range(H)])
    o, lse = block_sparse_attention(q, k, v, masks, bs)
    for b in range(B):
        for h in range(H):
            o1, l1 = block_sparse_attention_head(q[b, h], k[b, h], v[b, h], masks[h], bs)
            assert (o[b, h] == o1).all() and (lse[b, h] == l1).all()


# ----------------------------------------------------------------------------- backward


def _loss(q, k, v, g, mask, bs, causal):
    o, _ = block_sparse_attention_head(q, k, v, mask, bs, causal=causal)
    return float((g * o).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    rng = np.random.default_rng(8)
    N, d, bs = 24, 3, 8
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)
    q, k, v, g = (rng.standard_normal((N, d)) for _ in range(4))
    dq, dk, dv, _ = oracle.block_sparse_attention_backward_head(q, k, v, g, mask, bs,
                                                                causal=causal)
    eps = 1e-6
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = _loss(q, k, v, g, mask, bs, causal)
            x[idx] = x0 - eps
            lm = _loss(q, k, v, g, mask, bs, causal)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - grad).max() < 1e-7 * max(1.0, np.abs(grad).max())


def _sdpa_grads(q, k, v, g, attn_mask=None, is_causal=False):
    ts = [torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(
        *(t[None, None] for t in ts), attn_mask=attn_mask, is_causal=is_causal)[0, 0]
    (o * torch.from_numpy(g)).sum().backward()
    return [t.grad.numpy() for t in ts], o.detach().numpy()


@pytest.mark.parametrize("kind", ["ones", "causal", "mask"])
def test_backward_matches_sdpa_autograd(kind):
    rng = np.random.default_rng(9)
    N, d, bs = 128, 16, 32
    q, k, v, g = (rng.standard_normal((N, d)) for _ in range(4))
    if kind == "mask":
        mask = random_block_mask(4, 0.5, 3)
        token = torch.from_numpy(np.kron(mask, np.ones((bs, bs))) != 0)
        (gq, gk, gv), o = _sdpa_grads(q, k, v, g, attn_mask=token)
    else:
        mask = np.ones((4, 4), np.uint8)
        (gq, gk, gv), o = _sdpa_grads(q, k, v, g, is_causal=kind == "causal")
    dq, dk, dv, dvec = oracle.block_sparse_attention_backward_head(q, k, v, g, mask, bs,
                                                                   causal=kind == "causal")
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert np.abs(a - b).max() < 1e-12 * max(1.0, np.abs(b).max())
    assert np.abs(dvec - (g * o).sum(axis=1)).max() < 1e-12


# ----------------------------------------------------------------------------- decode


def _decode_visible(length, mask, bs):
    t = length - 1
    pos = np.arange(length)
    return mask[t // bs][pos // bs] != 0


@pytest.mark.parametrize("length", [1, 31, 32, 33, 100, 255, 256])
def test_decode_equals_masked_sdpa_on_the_prefix(length):
    rng = np.random.default_rng(length)
    n_cap, d, bs = 256, 16, 32
    q = rng.standard_normal(d)
    k, v = rng.standard_normal((n_cap, d)), rng.standard_normal((n_cap, d))
    mask = random_block_mask(n_cap // bs, 0.4, 11)
    o, lse = oracle.block_sparse_decode_head(q, k, v, length, mask, bs)
    vis = _decode_visible(length, mask, bs)
    ref = _sdpa(q[None], k[:length], v[:length], mask=vis[None])[0]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = (k[:length] @ q) / math.sqrt(d)
    assert abs(lse - logsumexp(s[vis])) < 1e-12


def test_decode_textbook_loop():
    rng = np.random.default_rng(3)
    n_cap, d, bs, length = 64, 4, 16, 40
    q, k, v = rng.standard_normal(d), rng.standard_normal((n_cap, d)), rng.standard_normal((n_cap, d))
    mask = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [1, 0, 1, 1], [0, 0, 0, 1]], np.uint8)
    # token 39 is in block 2, which selects blocks 0, 2 (and 3, all after it)
    num, den, mx = np.zeros(d), 0.0, -math.inf
    scores = [(p, float(q @ k[p]) * 0.5) for p in list(range(0, 16)) + list(range(32, 40))]
    mx = max(s for _, s in scores)
    for p, s in scores:
        w = math.exp(s - mx)
        num += w * v[p]
        den += w
    o, lse = oracle.block_sparse_decode_head(q, k, v, length, mask, bs)
    np.testing.assert_allclose(o, num / den, rtol=0, atol=1e-13)
    assert abs(lse - (mx + math.log(den))) < 1e-13


def test_decode_zero_query_is_uniform_over_visible_keys():
    rng = np.random.default_rng(4)
    n_cap, d, bs = 4096, 8, 32
    k, v = rng.standard_normal((n_cap, d)), rng.standard_normal((n_cap, d))
    sets = oracle.loglinear_block_sets(n_cap, bs)
    mask = block_mask_from_sets(sets)
    # worked-example pattern: the last token (block 127) selects {0, 64, 123, 125, 126, 127}
    o, lse = oracle.block_sparse_decode_head(np.zeros(d), k, v, n_cap, mask, bs)
    rows = np.concatenate([np.arange(j * bs, (j + 1) * bs) for j in (0, 64, 123, 125, 126, 127)])
    np.testing.assert_allclose(o, v[rows].mean(axis=0), rtol=0, atol=1e-12)
    assert abs(lse - math.log(6 * bs)) < 1e-12
    # a token in the middle of block 100 sees blocks {0, 64, 96, 98, 99} in full and
    # 17 keys of its own block
    length = 100 * bs + 17
    o, lse = oracle.block_sparse_decode_head(np.zeros(d), k, v, length, mask, bs)
    assert abs(lse - math.log(5 * bs + 17)) < 1e-12


def test_decode_token_without_visible_keys_and_bad_length():
    n_cap, d, bs = 64, 4, 16
    k = v = np.ones((n_cap, d))
    mask = np.eye(4, dtype=np.uint8)
    mask[2, 2] = 0
    mask[2, 3] = 1  # block 2 selects only a later block
    o, lse = oracle.block_sparse_decode_head(np.ones(d), k, v, 40, mask, bs)
    assert np.all(o == 0) and lse == -math.inf
    with pytest.raises(ValueError):
        oracle.block_sparse_decode_head(np.ones(d), k, v, 0, mask, bs)
    with pytest.raises(ValueError):
        oracle.block_sparse_decode_head(np.ones(d), k, v, n_cap + 1, mask, bs)


def test_decode_batched_wrapper_with_per_head_masks():
    rng = np.random.default_rng(5)
    B, H, n_cap, d, bs = 2, 3, 128, 8, 32
    q = rng.standard_normal((B, H, d))
    k, v = rng.standard_normal((B, H, n_cap, d)), rng.standard_normal((B, H, n_cap, d))
    masks = np.stack([random_block_mask(4, 0.5, s) for s in range(H)])
    lengths = [77, 128]
    o, lse = oracle.block_sparse_decode(q, k, v, lengths, masks, bs)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.block_sparse_decode_head(q[b, h], k[b, h], v[b, h], lengths[b],
                                                     masks[h], bs)
            assert np.array_equal(o[b, h], o1) and lse[b, h] == l1


# ----------------------------------------------------------------------------- int8 K/V


def test_quantize_closed_form_power_of_two_scale():
    # values k / 64, k = -127..127, with one element at 127 / 64: scale = 1/64
    # exactly and every code equals k
    bs, d = 32, 8
    rng = np.random.default_rng(0)
    k = rng.integers(-127, 128, size=(2, bs, d))
    k[0, 5, 3] = 127
    k[1, 0, 0] = -127
    x = (k / 64.0).reshape(2 * bs, d).astype(np.float32)
    codes, scales = oracle.quantize_blocks(x, bs)
    assert scales.dtype == np.float32 and np.all(scales == np.float32(1 / 64))
    assert np.array_equal(codes.reshape(2, bs, d), k.astype(np.int8))


def test_quantize_bounds_extremes_and_zero_block():
    bs, d = 16, 32
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 4 * bs, d)).astype(np.float32)
    x[1, bs:2 * bs] = 0.0  # an all-zero block
    codes, scales = oracle.quantize_blocks(x, bs)
    assert codes.dtype == np.int8 and scales.shape == (3, 4)
    assert np.abs(codes.astype(int)).max() <= 127
    assert scales[1, 1] == 0 and np.all(codes[1, bs:2 * bs] == 0)
    deq = oracle.dequantize_blocks(codes, scales, bs)
    step = np.repeat(scales, bs, axis=-1)[..., None].astype(np.float64)
    assert np.all(np.abs(deq - x) <= step / 2 * (1 + 1e-6))
    for b in range(3):
        for j in range(4):
            blk = x[b, j * bs:(j + 1) * bs]
            if scales[b, j] == 0:
                continue
            r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert abs(int(codes[b, j * bs + r, c])) == 127


def test_decode_int8_on_dequantised_cache_equals_masked_sdpa():
    rng = np.random.default_rng(2)
    n_cap, d, bs, length = 256, 16, 32, 201
    q = rng.standard_normal(d)
    k = rng.standard_normal((n_cap, d)).astype(np.float32)
    v = rng.standard_normal((n_cap, d)).astype(np.float32)
    kc, ks = oracle.quantize_blocks(k, bs)
    vc, vs = oracle.quantize_blocks(v, bs)
    mask = random_block_mask(n_cap // bs, 0.5, 4)
    o, lse = oracle.block_sparse_decode_int8(q[None, None], kc[None, None], ks[None, None],
                                             vc[None, None], vs[None, None], [length], mask, bs)
    kd = kc.astype(np.float64) * np.repeat(ks, bs)[:, None]
    vd = vc.astype(np.float64) * np.repeat(vs, bs)[:, None]
    vis = _decode_visible(length, mask, bs)
    ref = _sdpa(q[None], kd[:length], vd[:length], mask=vis[None])[0]
    np.testing.assert_allclose(o[0, 0], ref, rtol=0, atol=1e-12)
    s = (kd[:length] @ q) / math.sqrt(d)
    assert abs(lse[0, 0] - logsumexp(s[vis])) < 1e-12
