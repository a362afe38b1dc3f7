"""The C-ABI library loads, exports every symbol include/bsa.h declares, and
bsa_forward rejects bad arguments on the host before any HIP call (so these
run without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_csr_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared_functions()
    assert {"bsa_build_pattern", "bsa_forward", "bsa_status_string", "bsa_abi_version"} <= set(
        names)


def test_library_exports_every_declared_symbol():
    lib = bsa._load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_library_has_gfx950_code_object():
    # the library built here embeds a device code object for gfx950
    blob = open(bsa.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_abi_version_and_status_strings():
    assert bsa.abi_version() == 4
    for code in range(8):
        assert bsa.status_string(code).startswith("BSA_")
    assert bsa.status_string(99) == "BSA_ERR_UNKNOWN"


FAKE = 1 << 20  # a 16-byte-aligned non-null pointer value; never dereferenced


def _fwd(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=8, N=4096, d=64, bs=32,
                dtype=1, row_ptr=FAKE, col_idx=FAKE, nnz=1251, scale=0.0, stream=None)
    args.update(over)
    lib = bsa._load()
    return lib.bsa_forward(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                           args["H"], args["N"], args["d"], args["bs"], args["dtype"],
                           args["row_ptr"], args["col_idx"], args["nnz"],
                           ctypes.c_float(args["scale"]), args["stream"])


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "row_ptr", "col_idx"])
def test_forward_null_pointer(field):
    assert _fwd(**{field: None}) == 1


@pytest.mark.parametrize("over", [{"d": 96}, {"d": 32}, {"d": 256}, {"bs": 16}, {"bs": 128},
                                  {"dtype": 2}, {"dtype": -1}, {"q": FAKE + 2},
                                  {"o": FAKE + 8}, {"scale": float("nan")},
                                  {"scale": float("inf")}])
def test_forward_invalid_argument(over):
    assert _fwd(**over) == 2


@pytest.mark.parametrize("over", [{"B": 0}, {"H": -1}, {"N": 4010}, {"N": 0}, {"nnz": 127},
                                  {"nnz": 128 * 128 + 1}, {"B": 1 << 20, "H": 1 << 12}])
def test_forward_shape(over):
    assert _fwd(**over) == 3


def test_python_forward_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    rp = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):
        bsa.forward(q, q, q, rp, rp, 32)


def _fwd_ex(flags, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=8, N=4096, d=64, bs=32,
                dtype=1, row_ptr=FAKE, col_idx=FAKE, nnz=1251, scale=0.0, stream=None)
    args.update(over)
    lib = bsa._load()
    return lib.bsa_forward_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                              args["H"], args["N"], args["d"], args["bs"], args["dtype"],
                              args["row_ptr"], args["col_idx"], args["nnz"],
                              ctypes.c_float(args["scale"]), flags, 0, 0, args["stream"])


@pytest.mark.parametrize("flags", [4, 8, -1, 1 << 30])
def test_forward_ex_unknown_flags(flags):
    assert _fwd_ex(flags) == 2


def test_forward_ex_per_head_nnz_range():
    # 8 heads of M = 128: nnz must lie in [8 * 128, 8 * 128 * 128]
    assert _fwd_ex(2, nnz=8 * 128 - 1) == 3
    assert _fwd_ex(2, nnz=8 * 128 * 128 + 1) == 3
    assert _fwd_ex(3, nnz=1251, q=None) == 1


def test_forward_ex_bad_shape_flags_combination():
    assert _fwd_ex(1, d=96) == 2
    assert _fwd_ex(1, N=4010) == 3


def _dec(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=4, H=8, N=4096, d=64, bs=32,
                dtype=1, seqlens=FAKE, row_ptr=FAKE, col_idx=FAKE, nnz=1251, scale=0.0,
                flags=0, stream=None)
    args.update(over)
    a = args
    return bsa._load().bsa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                  a["N"], a["d"], a["bs"], a["dtype"], a["seqlens"],
                                  a["row_ptr"], a["col_idx"], a["nnz"],
                                  ctypes.c_float(a["scale"]), a["flags"], a["stream"])


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "seqlens", "row_ptr", "col_idx"])
def test_decode_null_pointer(field):
    assert _dec(**{field: None}) == 1


@pytest.mark.parametrize("over", [{"d": 96}, {"bs": 16}, {"dtype": 2}, {"k": FAKE + 4},
                                  {"scale": float("nan")}, {"flags": 1}, {"flags": 4}])
def test_decode_invalid_argument(over):
    assert _dec(**over) == 2


@pytest.mark.parametrize("over", [{"B": 0}, {"H": 0}, {"N": 4010}, {"nnz": 127},
                                  {"nnz": 128 * 128 + 1}, {"flags": 2, "nnz": 1000}])
def test_decode_shape_errors(over):
    # flags 2 (one pattern per head) needs heads * M <= nnz
    assert _dec(**over) == 3


def test_quantize_and_int8_decode_host_errors():
    lib = bsa._load()
    f = ctypes.c_float
    q = lambda **o: lib.bsa_quantize_kv(o.get("x", FAKE), o.get("codes", FAKE),
                                        o.get("scales", FAKE), o.get("B", 2), o.get("H", 4),
                                        o.get("N", 1024), o.get("d", 64), o.get("bs", 32),
                                        o.get("dtype", 1), None)
    assert q(x=None) == 1 and q(codes=None) == 1 and q(scales=None) == 1
    assert q(d=96) == 2 and q(bs=16) == 2 and q(dtype=3) == 2 and q(codes=FAKE + 8) == 2
    assert q(N=1000) == 3 and q(B=0) == 3
    d8 = lambda **o: lib.bsa_decode_int8kv(
        FAKE, FAKE, o.get("ks", FAKE), FAKE, o.get("vs", FAKE), FAKE, FAKE, 4, 8, 4096, 64, 32,
        1, FAKE, FAKE, FAKE, o.get("nnz", 1251), f(0.0), o.get("flags", 0), None)
    assert d8(ks=None) == 1 and d8(vs=None) == 1
    assert d8(flags=1) == 2 and d8(nnz=5) == 3


def _fwd_split(**over):
    """bsa_forward_split with a plan of 16 items over 2 heavy rows; every case
    below fails validation before any HIP call."""
    lib = bsa._load()
    need = lib.bsa_row_split_workspace_bytes(1, 8, 32, 64, 16)
    args = dict(flags=0, heavy=FAKE, items=FAKE, n_items=16, rows=FAKE, n_rows=2, ws=FAKE,
                ws_bytes=need, nnz=1251)
    args.update(over)
    return lib.bsa_forward_split(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4096, 64, 32, 1, FAKE, FAKE,
                                 args["nnz"], ctypes.c_float(0.0), args["flags"], args["heavy"],
                                 args["items"], args["n_items"], args["rows"], args["n_rows"],
                                 args["ws"], args["ws_bytes"], None)


def test_forward_split_rejects_bad_plans():
    assert _fwd_split(flags=2) == 2                  # one plan cannot serve per-head patterns
    assert _fwd_split(flags=4) == 2                  # unknown flag
    assert _fwd_split(n_rows=0) == 3                 # items without heavy rows
    assert _fwd_split(n_items=-1) == 3
    assert _fwd_split(n_rows=129) == 3               # more heavy rows than rows
    assert _fwd_split(n_items=1252) == 3             # more items than entries
    for field in ("heavy", "items", "rows", "ws"):
        assert _fwd_split(**{field: None}) == 1
    assert _fwd_split(ws=FAKE + 4) == 2              # workspace not 16-byte aligned
    lib = bsa._load()
    need = lib.bsa_row_split_workspace_bytes(1, 8, 32, 64, 16)
    assert _fwd_split(ws_bytes=need - 1) == 6        # workspace too small
    assert lib.bsa_row_split_workspace_bytes(0, 8, 32, 64, 16) == -1
    assert lib.bsa_row_split_workspace_bytes(1, 8, 32, 96, 16) == -1
