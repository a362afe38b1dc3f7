"""libbsa driven from a plain C program (tests/c/bsa_c_forward.c, built next
to the library), with no Python in that process.

CPU: the program's pattern mode -- bsa_build_pattern, bsa_transpose_pattern,
bsa_pattern_order and bsa_plan_row_split called from C -- against the oracle's
log-linear rule ([P1] "Block Sparse Attention: Log-Linear complexity sparse
attention implementation", section 3.1), the local + global block mask of
section 2.2, numpy transposes, and the order and split rules restated here.

GPU: the program's forward mode (bsa_forward in float32 through the HIP
runtime's C API) against the float64 oracle, element by element, at the
float32 bar ||O - O_ref||_inf / ||O_ref||_inf <= 1e-5 (same for LSE).
"""

import math
import os
import subprocess

import numpy as np
import pytest

import block_sparse_attention_csr_amd as bsa
import oracle
from synthetic_inputs import local_global_block_mask, make_qkv

PROGRAM = os.path.join(os.path.dirname(bsa.library_path()), "bsa_c_forward")
F32_RTOL = 1e-5


def _program():
    if not os.path.exists(PROGRAM):
        raise FileNotFoundError(f"{PROGRAM} is missing: run block_sparse_attention_csr_amd.build")
    return PROGRAM


def _parse(text):
    out = {}
    for line in text.splitlines():
        name, *vals = line.split()
        out[name] = np.array([int(v) for v in vals], dtype=np.int64)
    return out


def _order_rule(ptr):
    """Blocks with more than twice the mean count first (longest first, ties
    ascending), then the rest ascending."""
    cnt = np.diff(ptr)
    M = cnt.size
    long_ = [i for i in range(M) if cnt[i] * M > 2 * ptr[-1]]
    long_.sort(key=lambda i: (-cnt[i], i))
    return np.array(long_ + [i for i in range(M) if i not in set(long_)])


def _check_split(ptr, heavy, items, rows):
    """The default plan: chunk = mean row length rounded up to 8 (at least 8);
    heavy iff more than 2 * chunk entries; a heavy row's entries cut in order
    into items of at most chunk."""
    M = ptr.size - 1
    chunk = max(8, -(-math.ceil(ptr[-1] / M) // 8) * 8)
    cnt = np.diff(ptr)
    np.testing.assert_array_equal(heavy, (cnt > 2 * chunk).astype(np.int64))
    items = items.reshape(-1, 3)
    rows = rows.reshape(-1, 3)
    assert [r for r, _, _ in rows] == [i for i in range(M) if heavy[i]]
    for r, first, count in rows:
        its = items[first:first + count]
        assert count == -(-cnt[r] // chunk)
        assert (its[:, 0] == r).all()
        assert its[0, 1] == ptr[r] and its[-1, 2] == ptr[r + 1]
        assert (its[1:, 1] == its[:-1, 2]).all()
        assert (its[:, 2] - its[:, 1] <= chunk).all() and (its[:, 2] > its[:, 1]).all()
    assert sum(rows[:, 2]) == items.shape[0]


@pytest.mark.parametrize("N,bs", [(4096, 32), (8192, 64), (512, 32)])
def test_pattern_mode_matches_oracle(N, bs):
    r = subprocess.run([_program(), "pattern", str(N), str(bs)], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 0, r.stderr
    got = _parse(r.stdout)
    assert got["abi"][0] == bsa.abi_version()
    M = N // bs
    masks = {"": oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs)),
             "lg_": local_global_block_mask(M)}
    for pre, mask in masks.items():
        rp, ci = oracle.csr_from_block_mask(mask)
        cp, ri = oracle.csr_from_block_mask(np.ascontiguousarray(mask.T))
        assert got[pre + "M"][0] == M and got[pre + "nnz"][0] == rp[-1]
        np.testing.assert_array_equal(got[pre + "row_ptr"], rp)
        np.testing.assert_array_equal(got[pre + "col_idx"], ci)
        np.testing.assert_array_equal(got[pre + "col_ptr"], cp)
        np.testing.assert_array_equal(got[pre + "row_idx"], ri)
        np.testing.assert_array_equal(got[pre + "row_order"], _order_rule(np.asarray(rp)))
        np.testing.assert_array_equal(got[pre + "col_order"], _order_rule(np.asarray(cp)))
        _check_split(np.asarray(rp, dtype=np.int64), got[pre + "heavy"], got[pre + "items"],
                     got[pre + "split_rows"])
    # at M = 128 and above the local + global rows are long enough to split
    if M >= 128:
        assert got["lg_heavy"][0] == 1 and got["lg_heavy"][M - 1] == 1
        assert got["lg_split_rows"].size == 6


@pytest.mark.parametrize("argv,code,text", [
    (["pattern", "4010", "32"], 2, "BSA_ERR_SHAPE"),
    (["pattern", "4096", "0"], 2, "BSA_ERR_"),
    (["forward", "/nonexistent/in.bin", "/nonexistent/out.bin"], 1, "cannot open"),
    ([], 1, "usage"),
])
def test_program_reports_errors(argv, code, text):
    r = subprocess.run([_program(), *argv], capture_output=True, text=True, timeout=60)
    assert r.returncode == code
    assert text in r.stderr


def test_forward_mode_rejects_bad_header(tmp_path):
    # sizes are checked before any HIP call, so this runs without a GPU
    inp = tmp_path / "in.bin"
    np.array([1, 1, 4010, 64, 32], dtype=np.int32).tofile(inp)
    r = subprocess.run([_program(), "forward", str(inp), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "bad sizes" in r.stderr
    np.array([1, 1, 64, 64, 32], dtype=np.int32).tofile(inp)  # header only, no data
    r = subprocess.run([_program(), "forward", str(inp), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "short data" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,N,d,bs", [(1, 2, 1024, 64, 32), (2, 1, 2048, 128, 64),
                                        (1, 1, 4096, 64, 32)])
def test_forward_mode_matches_oracle(tmp_path, B, H, N, d, bs):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = make_qkv(B, H, N, d, dtype=torch.float32, seed=N + d)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([B, H, N, d, bs], dtype=np.int32).tobytes())
        for t in (q, k, v):
            f.write(t.numpy().astype(np.float32).tobytes())
    print(f"bsa_c_forward forward B={B} H={H} N={N} d={d} bs={bs}", flush=True)
    r = subprocess.run([_program(), "forward", str(inp), str(outp)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(outp, dtype=np.float32)
    n_x = B * H * N * d
    assert raw.size == n_x + B * H * N
    o = raw[:n_x].reshape(B, H, N, d).astype(np.float64)
    lse = raw[n_x:].reshape(B, H, N).astype(np.float64)
    mask = oracle.block_mask_from_sets(oracle.loglinear_block_sets(N, bs))
    o_ref, lse_ref = oracle.block_sparse_attention(q.double().numpy(), k.double().numpy(),
                                                   v.double().numpy(), mask, bs)
    assert np.abs(o - o_ref).max() <= F32_RTOL * np.abs(o_ref).max()
    assert np.abs(lse - lse_ref).max() <= F32_RTOL * np.abs(lse_ref).max()
