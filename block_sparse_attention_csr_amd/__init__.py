"""Block-sparse attention forward for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libbsa.so`` (declared in
``include/bsa.h``): argument marshalling only.  Every step of the attention
runs in the native library: the pattern builder on the host, the forward in
one HIP kernel.  PyTorch provides device memory and the current stream.

    row_ptr, col_idx = build_pattern(4096, 32)                 # log-linear rule
    row_ptr, col_idx = build_pattern(4096, 64, mask=block_mask)  # user mask
    o, lse = forward(q, k, v, row_ptr.cuda(), col_idx.cuda(), block_size=32)

There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "BsaError", "build_pattern", "forward", "backward", "transpose_pattern", "status_string",
    "abi_version", "library_path", "PatternCache", "BSA_OK", "stack_head_patterns",
    "pattern_order", "decode", "quantize_kv", "decode_int8kv", "attention", "plan_row_split",
    "RowSplitPlan", "backward_noalloc", "forward_int8kv",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libbsa.so")

BSA_OK = 0
_PATTERN_LOGLINEAR = 0
_PATTERN_BLOCK_MASK = 1
_PATTERN_DILATED = 2
_PATTERN_BIGBIRD = 3
FORWARD_CAUSAL = 1
FORWARD_PATTERN_PER_HEAD = 2
_DTYPE_F32 = 0
_DTYPE_BF16 = 1


class BsaError(RuntimeError):
    """A bsa_* call returned a status other than BSA_OK."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _PatternDesc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("local_radius", ctypes.c_int32),
        ("k_max", ctypes.c_int32),
        ("num_global", ctypes.c_int32),
        ("global_blocks", ctypes.POINTER(ctypes.c_int32)),
        ("mask", ctypes.POINTER(ctypes.c_uint8)),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dilation", ctypes.c_int32),
        ("num_random", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"native library not built: {_LIB_PATH} is missing "
            "(run `python -m block_sparse_attention_csr_amd.build`)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.bsa_build_pattern.argtypes = [ctypes.POINTER(_PatternDesc), p32, p32, i64,
                                      ctypes.POINTER(i64)]
    lib.bsa_build_pattern.restype = i32
    lib.bsa_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i64,
                                ctypes.c_float, vp]
    lib.bsa_forward.restype = i32
    lib.bsa_forward_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                   i64, ctypes.c_float, i32, i32, i32, vp]
    lib.bsa_forward_ex.restype = i32
    p8 = ctypes.POINTER(ctypes.c_uint8)
    lib.bsa_plan_row_split.argtypes = [i32, p32, i32, p8, p32, i32, p32, p32, p32]
    lib.bsa_plan_row_split.restype = i32
    lib.bsa_row_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.bsa_row_split_workspace_bytes.restype = i64
    lib.bsa_forward_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                      i64, ctypes.c_float, i32, vp, vp, i32, vp, i32, vp, i64,
                                      vp]
    lib.bsa_forward_split.restype = i32
    lib.bsa_transpose_pattern.argtypes = [i32, p32, p32, i64, p32, p32]
    lib.bsa_transpose_pattern.restype = i32
    lib.bsa_backward.argtypes = [vp] * 10 + [i32] * 6 + [vp] * 6 + [i64, ctypes.c_float, i32, vp]
    lib.bsa_forward_int8kv.argtypes = ([vp] * 7 + [i32] * 5 + [vp, vp, i64, ctypes.c_float]
                                       + [i32] * 3 + [vp])
    lib.bsa_forward_int8kv.restype = i32
    lib.bsa_backward_noalloc.argtypes = ([vp] * 9 + [i32] * 6 + [vp] * 6
                                         + [i64, ctypes.c_float, i32, vp])
    lib.bsa_backward_noalloc.restype = i32
    lib.bsa_backward_noalloc_max_rows.argtypes = []
    lib.bsa_backward_noalloc_max_rows.restype = i64
    lib.bsa_pattern_order.argtypes = [i32, p32, p32]
    lib.bsa_pattern_order.restype = i32
    lib.bsa_backward.restype = i32
    lib.bsa_decode.argtypes = [vp] * 5 + [i32] * 6 + [vp] * 3 + [i64, ctypes.c_float, i32, vp]
    lib.bsa_decode.restype = i32
    lib.bsa_quantize_kv.argtypes = [vp] * 3 + [i32] * 6 + [vp]
    lib.bsa_quantize_kv.restype = i32
    lib.bsa_decode_int8kv.argtypes = [vp] * 7 + [i32] * 6 + [vp] * 3 + [i64, ctypes.c_float,
                                                                          i32, vp]
    lib.bsa_decode_int8kv.restype = i32
    lib.bsa_status_string.argtypes = [i32]
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_abi_version.argtypes = []
    lib.bsa_abi_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return _load().bsa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_load().bsa_abi_version())


def _desc(seq_len, block_size, kind, mask, local_radius, k_max, global_blocks, causal, window,
          dilation, num_random, seed, keep):
    d = _PatternDesc()
    d.seq_len = int(seq_len)
    d.block_size = int(block_size)
    d.local_radius = -1 if local_radius is None else int(local_radius)
    d.k_max = -1 if k_max is None else int(k_max)
    d.num_global = -1
    d.global_blocks = None
    d.mask = None
    d.causal = 1 if causal else 0
    d.window = 0 if window is None else int(window)
    d.dilation = 1 if dilation is None else int(dilation)
    d.num_random = 0 if num_random is None else int(num_random)
    d.seed = 0 if seed is None else int(seed) & ((1 << 64) - 1)
    if kind is None:
        kind = "mask" if mask is not None else "loglinear"
    codes = {"loglinear": _PATTERN_LOGLINEAR, "mask": _PATTERN_BLOCK_MASK,
             "dilated": _PATTERN_DILATED, "bigbird": _PATTERN_BIGBIRD}
    if kind not in codes:
        raise ValueError(f"unknown pattern kind {kind!r}; one of {sorted(codes)}")
    d.kind = codes[kind]
    if kind == "mask":
        if mask is None:
            raise ValueError("kind 'mask' needs a mask")
        m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
        keep.append(m)
        d.mask = m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    elif global_blocks is not None:
        g = np.ascontiguousarray(np.asarray(global_blocks, dtype=np.int32).reshape(-1))
        keep.append(g)
        d.num_global = int(g.size)
        d.global_blocks = g.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return d


def build_pattern(seq_len: int, block_size: int, *, mask=None, local_radius=None, k_max=None,
                  global_blocks=None, causal: bool = False, kind: str | None = None,
                  window: int | None = None, dilation: int | None = None,
                  num_random: int | None = None, seed: int | None = None):
    """CSR (row_ptr int32[M+1], col_idx int32[nnz]) as CPU torch tensors.

    ``kind``: "loglinear" (default without ``mask``: radius 1,
    k_max = ceil(log2 M), globals {0, M/2, M-1}), "mask" (default with
    ``mask``: an [M, M] array, nonzero = selected), "dilated" (``window``,
    ``dilation``, optional ``global_blocks``) or "bigbird" (``local_radius``,
    ``global_blocks``, ``num_random`` per row drawn from ``seed``).
    ``causal`` drops blocks after each query block.  Raises BsaError on a bad
    pattern.
    """
    import torch

    lib = _load()
    keep = []
    desc = _desc(seq_len, block_size, kind, mask, local_radius, k_max, global_blocks, causal,
                 window, dilation, num_random, seed, keep)
    nnz = ctypes.c_int64(0)
    st = lib.bsa_build_pattern(ctypes.byref(desc), None, None, 0, ctypes.byref(nnz))
    if st != BSA_OK:
        raise BsaError(st, "bsa_build_pattern")
    M = seq_len // block_size
    row_ptr = np.zeros(M + 1, dtype=np.int32)
    col_idx = np.zeros(max(nnz.value, 1), dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = lib.bsa_build_pattern(ctypes.byref(desc), row_ptr.ctypes.data_as(p32),
                               col_idx.ctypes.data_as(p32), col_idx.size, ctypes.byref(nnz))
    if st != BSA_OK:
        raise BsaError(st, "bsa_build_pattern")
    return torch.from_numpy(row_ptr), torch.from_numpy(col_idx[:nnz.value].copy())


def stack_head_patterns(patterns):
    """One CSR per head -> (row_ptr int32[H*(M+1)], col_idx int32[nnz]) for the
    per-head forward: head h's row offsets are shifted by the entries of the
    heads before it, so that they index the one concatenated col_idx."""
    import torch

    rps, cis = [], []
    base = 0
    for row_ptr, col_idx in patterns:
        rps.append(row_ptr.to(torch.int64) + base)
        cis.append(col_idx)
        base += int(col_idx.numel())
    if base > 2**31 - 1:
        raise ValueError("per-head patterns exceed int32 offsets")
    return torch.cat(rps).to(torch.int32), torch.cat(cis).to(torch.int32)


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return _DTYPE_BF16
    if t.dtype == torch.float32:
        return _DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; bfloat16 or float32 expected")


class RowSplitPlan:
    """A bsa_plan_row_split plan: ``heavy`` uint8 [M], ``items`` int32
    [n_items, 3] (row, first entry, end entry) and ``rows`` int32 [n_rows, 3]
    (row, first item, item count), on the CPU or (``to``) on a device."""

    def __init__(self, heavy, items, rows):
        self.heavy, self.items, self.rows = heavy, items, rows
        self.n_items = int(items.shape[0])
        self.n_rows = int(rows.shape[0])

    def to(self, device):
        return RowSplitPlan(self.heavy.to(device), self.items.to(device), self.rows.to(device))


def plan_row_split(row_ptr, chunk: int = 0):
    """bsa_plan_row_split of a host CSR's offsets: a RowSplitPlan (CPU
    tensors), or None when no row is long enough to split."""
    import torch

    pt = np.ascontiguousarray(np.asarray(row_ptr.cpu() if hasattr(row_ptr, "cpu") else row_ptr,
                                         dtype=np.int32))
    M = pt.size - 1
    cap = max(int(pt[-1]), 1)
    heavy = np.zeros(max(M, 1), np.uint8)
    items = np.zeros(3 * cap, np.int32)
    rows = np.zeros(3 * max(M, 1), np.int32)
    n_items, n_rows = ctypes.c_int32(0), ctypes.c_int32(0)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = _load().bsa_plan_row_split(M, pt.ctypes.data_as(p32), int(chunk),
                                    heavy.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                    items.ctypes.data_as(p32), cap, ctypes.byref(n_items),
                                    rows.ctypes.data_as(p32), ctypes.byref(n_rows))
    if st != BSA_OK:
        raise BsaError(st, "bsa_plan_row_split")
    if n_items.value == 0:
        return None
    return RowSplitPlan(torch.from_numpy(heavy[:M].copy()),
                        torch.from_numpy(items[:3 * n_items.value].reshape(-1, 3).copy()),
                        torch.from_numpy(rows[:3 * n_rows.value].reshape(-1, 3).copy()))


def _on_stream(stream):
    """Context in which new tensors belong to ``stream`` in torch's caching
    allocator.  A buffer allocated on another stream and dropped when the
    call returns (a workspace, ``delta``) could otherwise be handed to new
    work while the kernels enqueued on ``stream`` still use it."""
    import torch

    return torch.cuda.stream(stream)


def _check_buffer(t, name, shape, dtype, device):
    """A caller-supplied device buffer: the library writes or reads it through
    a raw pointer, so its size, type and place are checked here."""
    if (not t.is_cuda or t.device != device or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def _check_csr(row_ptr, col_idx, device, rows, nnz, names=("row_ptr", "col_idx")):
    """Device CSR arrays: int32 on the device, `rows` + 1 offsets (the kernels
    read row_ptr[0 .. rows]) and at least nnz entries."""
    import torch

    for name, t in zip(names, (row_ptr, col_idx)):
        if t.dtype != torch.int32 or not t.is_cuda or t.device != device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor on {device}")
    if rows is not None and row_ptr.numel() != rows + 1:
        raise ValueError(f"{names[0]} must hold {rows + 1} offsets, not {row_ptr.numel()}")
    if col_idx.numel() < nnz:
        raise ValueError(f"{names[1]} holds {col_idx.numel()} entries, fewer than nnz = {nnz}")


def _pattern_rows(N: int, block_size: int, heads: int, per_head: bool):
    """Offsets minus one that row_ptr must hold, or None when the shape is
    invalid anyway (the library then reports it)."""
    if block_size <= 0 or N % block_size != 0:
        return None
    M = N // block_size
    return heads * (M + 1) - 1 if per_head else M


def forward(q, k, v, row_ptr, col_idx, block_size: int, scale: float | None = None, *,
            out=None, lse=None, nnz: int | None = None, stream=None, group: int = 0,
            key_split: int = 0, causal: bool = False, per_head: bool = False, split=None,
            workspace=None):
    """Block-sparse attention forward on the GPU.

    q, k, v: CUDA tensors [B, H, N, d] (bfloat16 or float32), contiguous.
    row_ptr, col_idx: int32 CUDA tensors from ``build_pattern`` (same device).
    Returns (o [B, H, N, d] same dtype, lse [B, H, N] float32).  The launch is
    enqueued on the current stream (or ``stream``) and not synchronised.
    ``nnz`` (host int) avoids reading row_ptr back; by default it is
    col_idx.numel().  ``group`` / ``key_split`` force a workgroup shape
    (bsa_forward_ex); 0 / 0 lets the library choose.  ``causal`` hides keys
    after each query position; ``per_head`` takes row_ptr as [H, M + 1]
    offsets into one col_idx (see ``stack_head_patterns``).  ``split``: a
    RowSplitPlan of the same pattern on the device (``plan_row_split``): its
    heavy rows are spread over workgroups (bsa_forward_split); ``workspace``
    optionally supplies the device bytes it needs, else they are allocated.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise TypeError("row_ptr / col_idx must be int32")
    if not (row_ptr.is_cuda and col_idx.is_cuda):
        raise ValueError("row_ptr / col_idx must be on the GPU")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if nnz is None:
        nnz = col_idx.numel()
    _check_csr(row_ptr, col_idx, q.device, _pattern_rows(N, int(block_size), H, per_head),
               int(nnz))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        with _on_stream(stream):
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    lib = _load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N,
            d, int(block_size), _dtype_code(q), row_ptr.data_ptr(), col_idx.data_ptr(),
            int(nnz), 0.0 if scale is None else float(scale))
    flags = (FORWARD_CAUSAL if causal else 0) | (FORWARD_PATTERN_PER_HEAD if per_head else 0)
    if split is not None:
        if group or key_split or per_head:
            raise ValueError("a row-split plan takes the automatic shape and one shared pattern")
        M = N // int(block_size) if int(block_size) > 0 else 0
        _check_buffer(split.heavy, "split.heavy", (M,), torch.uint8, q.device)
        _check_buffer(split.items, "split.items", (split.n_items, 3), torch.int32, q.device)
        _check_buffer(split.rows, "split.rows", (split.n_rows, 3), torch.int32, q.device)
        need = int(lib.bsa_row_split_workspace_bytes(B, H, int(block_size), d, split.n_items))
        if need < 0:
            raise ValueError("unsupported shape for a row-split plan")
        if workspace is None:
            with _on_stream(stream):
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        elif (not workspace.is_cuda or workspace.device != q.device
              or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < need):
            raise ValueError(f"workspace must be a contiguous tensor of >= {need} bytes on {q.device}")
        st = lib.bsa_forward_split(*args, flags, split.heavy.data_ptr(), split.items.data_ptr(),
                                   split.n_items, split.rows.data_ptr(), split.n_rows,
                                   workspace.data_ptr(), need, stream.cuda_stream)
        if st != BSA_OK:
            raise BsaError(st, "bsa_forward_split")
        return out, lse
    if group or key_split or flags:
        st = lib.bsa_forward_ex(*args, flags, int(group), int(key_split), stream.cuda_stream)
    else:
        st = lib.bsa_forward(*args, stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_forward")
    return out, lse


def forward_int8kv(q, k_codes, k_scales, v_codes, v_scales, row_ptr, col_idx, block_size: int,
                   scale: float | None = None, *, out=None, lse=None, nnz: int | None = None,
                   stream=None, group: int = 0, key_split: int = 0, causal: bool = False,
                   per_head: bool = False):
    """``forward`` on int8 K/V with per-block scales (bsa_forward_int8kv).

    q: bfloat16 CUDA [B, H, N, d]; k_codes, v_codes: int8 [B, H, N, d];
    k_scales, v_scales: float32 [B, H, N / block_size] (as ``quantize_kv``
    writes them).  Returns (o bfloat16 [B, H, N, d], lse float32 [B, H, N]).
    """
    import torch

    if not q.is_cuda or not q.is_contiguous() or q.dim() != 4 or q.dtype != torch.bfloat16:
        raise ValueError("q must be a contiguous bfloat16 CUDA tensor [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        _check_buffer(t, name, q.shape, torch.int8, q.device)
    if int(block_size) <= 0 or N % int(block_size) != 0:
        raise ValueError("N must be a positive multiple of block_size")
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        _check_buffer(t, name, (B, H, N // int(block_size)), torch.float32, q.device)
    if nnz is None:
        nnz = col_idx.numel()
    _check_csr(row_ptr, col_idx, q.device, _pattern_rows(N, int(block_size), H, per_head),
               int(nnz))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        with _on_stream(stream):
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    flags = (FORWARD_CAUSAL if causal else 0) | (FORWARD_PATTERN_PER_HEAD if per_head else 0)
    st = _load().bsa_forward_int8kv(
        q.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(),
        v_scales.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, int(block_size),
        row_ptr.data_ptr(), col_idx.data_ptr(), int(nnz), 0.0 if scale is None else float(scale),
        flags, int(group), int(key_split), stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_forward_int8kv")
    return out, lse


def transpose_pattern(row_ptr, col_idx):
    """CSC of a CSR pattern (bsa_transpose_pattern): (col_ptr int32[M+1],
    row_idx int32[nnz]) as CPU torch tensors; inputs are CPU int32 tensors."""
    import torch

    rp = np.ascontiguousarray(np.asarray(row_ptr.cpu() if hasattr(row_ptr, "cpu") else row_ptr,
                                         dtype=np.int32))
    ci = np.ascontiguousarray(np.asarray(col_idx.cpu() if hasattr(col_idx, "cpu") else col_idx,
                                         dtype=np.int32))
    M = rp.size - 1
    cp = np.zeros(M + 1, dtype=np.int32)
    ri = np.zeros(max(ci.size, 1), dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = _load().bsa_transpose_pattern(M, rp.ctypes.data_as(p32), ci.ctypes.data_as(p32),
                                       ci.size, cp.ctypes.data_as(p32), ri.ctypes.data_as(p32))
    if st != BSA_OK:
        raise BsaError(st, "bsa_transpose_pattern")
    return torch.from_numpy(cp), torch.from_numpy(ri[:ci.size].copy())


def pattern_order(ptr):
    """bsa_pattern_order: a work order for the blocks of a CSR row_ptr (or
    CSC col_ptr) -- blocks with more than twice the mean entry count first,
    longest first, then the rest ascending -- as a CPU int32 tensor of M."""
    import torch

    pt = np.ascontiguousarray(np.asarray(ptr.cpu() if hasattr(ptr, "cpu") else ptr,
                                         dtype=np.int32))
    M = pt.size - 1
    order = np.zeros(max(M, 1), dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = _load().bsa_pattern_order(M, pt.ctypes.data_as(p32), order.ctypes.data_as(p32))
    if st != BSA_OK:
        raise BsaError(st, "bsa_pattern_order")
    return torch.from_numpy(order[:M].copy())


def backward(q, k, v, o, lse, dout, row_ptr, col_idx, col_ptr, row_idx, block_size: int,
             scale: float | None = None, *, causal: bool = False, dq=None, dk=None, dv=None,
             delta=None, stream=None, row_order=None, col_order=None, per_head: bool = False):
    """Gradients (dq, dk, dv) of ``forward`` for the upstream gradient ``dout``.

    q, k, v, o, dout: CUDA [B, H, N, d] tensors of one dtype; lse the
    forward's LSE; row_ptr/col_idx the forward's device CSR and
    col_ptr/row_idx its device CSC (``transpose_pattern``); row_order /
    col_order optional device copies of ``pattern_order`` of the two (the
    blocks are then taken longest first).  ``per_head``: row_ptr and col_ptr
    are [H, M + 1] (``stack_head_patterns`` of each head's CSR, and of each
    head's ``transpose_pattern``); no orders then.  Enqueued on the current
    stream (or ``stream``), not synchronised.
    """
    import torch

    if not q.is_cuda or q.dim() != 4:
        raise ValueError("q must be a CUDA tensor [B, H, N, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_buffer(t, name, q.shape, q.dtype, q.device)
    B, H, N, d = q.shape
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    rows = _pattern_rows(N, int(block_size), H, per_head)
    _check_csr(row_ptr, col_idx, q.device, rows, col_idx.numel())
    _check_csr(col_ptr, row_idx, q.device, rows, col_idx.numel(), ("col_ptr", "row_idx"))
    if per_head and (row_order is not None or col_order is not None):
        raise ValueError("work orders are of one shared pattern: none with per_head")
    for t in (row_order, col_order):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda
                              or t.numel() != row_ptr.numel() - 1):
            raise ValueError("row_order / col_order must be int32 CUDA tensors of M entries")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _check_buffer(t, name, q.shape, q.dtype, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with _on_stream(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        if delta is None:
            delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        else:
            _check_buffer(delta, "delta", (B, H, N), torch.float32, q.device)
    st = _load().bsa_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d,
        int(block_size), _dtype_code(q), row_ptr.data_ptr(), col_idx.data_ptr(),
        col_ptr.data_ptr(), row_idx.data_ptr(),
        None if row_order is None else row_order.data_ptr(),
        None if col_order is None else col_order.data_ptr(), int(col_idx.numel()),
        0.0 if scale is None else float(scale),
        (FORWARD_CAUSAL if causal else 0) | (FORWARD_PATTERN_PER_HEAD if per_head else 0),
        stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_backward")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, dout, row_ptr, col_idx, col_ptr, row_idx,
                     block_size: int, dq, dk, dv, scale: float | None = None, *,
                     causal: bool = False, stream=None, row_order=None, col_order=None,
                     per_head: bool = False):
    """``backward`` through bsa_backward_noalloc: the caller passes dq, dk
    and dv, and D goes to the library's static device scratch instead of a
    workspace, so the call allocates nothing on the device.  Calls that
    overlap on one GPU share that scratch and must be ordered by the caller."""
    import torch

    if not q.is_cuda or q.dim() != 4:
        raise ValueError("q must be a CUDA tensor [B, H, N, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_buffer(t, name, q.shape, q.dtype, q.device)
    B, H, N, d = q.shape
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    rows = _pattern_rows(N, int(block_size), H, per_head)
    _check_csr(row_ptr, col_idx, q.device, rows, col_idx.numel())
    _check_csr(col_ptr, row_idx, q.device, rows, col_idx.numel(), ("col_ptr", "row_idx"))
    if per_head and (row_order is not None or col_order is not None):
        raise ValueError("work orders are of one shared pattern: none with per_head")
    for t in (row_order, col_order):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda
                              or t.numel() != row_ptr.numel() - 1):
            raise ValueError("row_order / col_order must be int32 CUDA tensors of M entries")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = _load().bsa_backward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, int(block_size), _dtype_code(q),
        row_ptr.data_ptr(), col_idx.data_ptr(), col_ptr.data_ptr(), row_idx.data_ptr(),
        None if row_order is None else row_order.data_ptr(),
        None if col_order is None else col_order.data_ptr(), int(col_idx.numel()),
        0.0 if scale is None else float(scale),
        (FORWARD_CAUSAL if causal else 0) | (FORWARD_PATTERN_PER_HEAD if per_head else 0),
        stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_backward_noalloc")
    return dq, dk, dv


def _decode_common(q, seqlens, row_ptr, col_idx, n_cap, block_size, per_head, nnz, out, lse,
                   stream):
    """Checks shared by the decode entry points; returns (out, lse), new ones
    allocated on ``stream``."""
    import torch

    B, H, d = q.shape
    if (seqlens.dtype != torch.int32 or not seqlens.is_cuda or seqlens.device != q.device
            or not seqlens.is_contiguous() or seqlens.numel() != B):
        raise ValueError(f"seqlens must be a contiguous int32 tensor of {B} entries on {q.device}")
    _check_csr(row_ptr, col_idx, q.device, _pattern_rows(n_cap, block_size, H, per_head), nnz)
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        with _on_stream(stream):
            lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, "lse", (B, H), torch.float32, q.device)
    return out, lse


def decode(q, k_cache, v_cache, seqlens, row_ptr, col_idx, block_size: int,
           scale: float | None = None, *, per_head: bool = False, out=None, lse=None,
           nnz: int | None = None, stream=None):
    """One new token per sequence against a block-aligned KV cache (bsa_decode).

    q: CUDA [B, H, d]; k_cache, v_cache: CUDA [B, H, N_cap, d] of q's dtype,
    contiguous; seqlens: int32 CUDA [B], each sequence's cached length L_b
    (the new token, already in the cache, is at position L_b - 1).
    row_ptr/col_idx: the device CSR of a pattern with N_cap / block_size rows
    (``per_head``: row_ptr [H, M + 1]).  Returns (o [B, H, d], lse [B, H]
    float32); enqueued on the current stream (or ``stream``), not synchronised.
    """
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, H, d] and the caches [B, H, N_cap, d]")
    B, H, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[1] != H or k_cache.shape[3] != d:
        raise ValueError("q and the caches disagree on B, H or d")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share a dtype")
    if k_cache.device != q.device or v_cache.device != q.device:
        raise ValueError("q and the caches must be on one device")
    n_cap = k_cache.shape[2]
    if nnz is None:
        nnz = col_idx.numel()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    out, lse = _decode_common(q, seqlens, row_ptr, col_idx, n_cap, int(block_size), per_head,
                              int(nnz), out, lse, stream)
    st = _load().bsa_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, H, n_cap, d, int(block_size), _dtype_code(q), seqlens.data_ptr(),
        row_ptr.data_ptr(), col_idx.data_ptr(), int(nnz), 0.0 if scale is None else float(scale),
        FORWARD_PATTERN_PER_HEAD if per_head else 0, stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_decode")
    return out, lse


def quantize_kv(x, block_size: int, *, codes=None, scales=None, stream=None):
    """int8 codes and per-block float32 scales of a CUDA [B, H, N, d] tensor
    (bsa_quantize_kv): returns (codes int8 [B, H, N, d], scales [B, H, N / bs])."""
    import torch

    if not x.is_cuda or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous CUDA tensor [B, H, N, d]")
    B, H, N, d = x.shape
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    if codes is None:
        with _on_stream(stream):
            codes = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    else:
        _check_buffer(codes, "codes", x.shape, torch.int8, x.device)
    if scales is None:
        with _on_stream(stream):
            scales = torch.empty((B, H, N // block_size), dtype=torch.float32, device=x.device)
    else:
        _check_buffer(scales, "scales", (B, H, N // block_size), torch.float32, x.device)
    st = _load().bsa_quantize_kv(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, d,
                                 int(block_size), _dtype_code(x), stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_quantize_kv")
    return codes, scales


def decode_int8kv(q, k_codes, k_scales, v_codes, v_scales, seqlens, row_ptr, col_idx,
                  block_size: int, scale: float | None = None, *, per_head: bool = False,
                  out=None, lse=None, nnz: int | None = None, stream=None):
    """``decode`` on an int8 KV cache with per-block scales (bsa_decode_int8kv):
    caches int8 [B, H, N_cap, d] and scales float32 [B, H, N_cap / bs] as
    ``quantize_kv`` writes them; q [B, H, d] bfloat16 or float32."""
    import torch

    if q.dim() != 3 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous CUDA tensor [B, H, d]")
    B, H, d = q.shape
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        if t.dtype != torch.int8 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous int8 CUDA tensor [B, H, N_cap, d]")
        if t.shape[0] != B or t.shape[1] != H or t.shape[3] != d:
            raise ValueError(f"{name} disagrees with q on B, H or d")
    n_cap = k_codes.shape[2]
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        if t.device != q.device or t.shape != k_codes.shape:
            raise ValueError("q and the code caches must be on one device, the caches alike")
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        _check_buffer(t, name, (B, H, n_cap // block_size), torch.float32, q.device)
    if nnz is None:
        nnz = col_idx.numel()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    out, lse = _decode_common(q, seqlens, row_ptr, col_idx, n_cap, int(block_size), per_head,
                              int(nnz), out, lse, stream)
    st = _load().bsa_decode_int8kv(
        q.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(),
        v_scales.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, n_cap, d, int(block_size),
        _dtype_code(q), seqlens.data_ptr(), row_ptr.data_ptr(), col_idx.data_ptr(), int(nnz),
        0.0 if scale is None else float(scale), FORWARD_PATTERN_PER_HEAD if per_head else 0,
        stream.cuda_stream)
    if st != BSA_OK:
        raise BsaError(st, "bsa_decode_int8kv")
    return out, lse


def attention(q, k, v, row_ptr, col_idx, col_ptr, row_idx, block_size: int,
              scale: float | None = None, *, causal: bool = False, row_order=None,
              col_order=None, per_head: bool = False):
    """Block-sparse attention as a differentiable torch operation: ``forward``
    on the way in, ``backward`` (with the saved O and LSE) on the way back.
    The pattern tensors are device int32 CSR / CSC (and optional work orders,
    see ``pattern_order``).  Returns O."""
    return _Attention.apply(q, k, v, row_ptr, col_idx, col_ptr, row_idx, int(block_size),
                            scale, bool(causal), row_order, col_order, bool(per_head))


def _make_attention_fn():
    import torch

    class _AttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, row_ptr, col_idx, col_ptr, row_idx, block_size, scale, causal,
                    row_order, col_order, per_head):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            o, lse = forward(q, k, v, row_ptr, col_idx, block_size, scale, causal=causal,
                             per_head=per_head)
            ctx.save_for_backward(q, k, v, o, lse, row_ptr, col_idx, col_ptr, row_idx)
            ctx.cfg = (block_size, scale, causal, row_order, col_order, per_head)
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse, row_ptr, col_idx, col_ptr, row_idx = ctx.saved_tensors
            block_size, scale, causal, row_order, col_order, per_head = ctx.cfg
            dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), row_ptr, col_idx, col_ptr,
                                  row_idx, block_size, scale, causal=causal,
                                  row_order=row_order, col_order=col_order, per_head=per_head)
            return dq, dk, dv, None, None, None, None, None, None, None, None, None, None

    return _AttentionFn


class _LazyAttention:
    fn = None

    @classmethod
    def apply(cls, *args):
        if cls.fn is None:
            cls.fn = _make_attention_fn()
        return cls.fn.apply(*args)


_Attention = _LazyAttention


class PatternCache:
    """Device-resident CSR patterns keyed by their descriptor.

    A model reuses one pattern for every layer and step at a given
    (seq_len, block_size); the host build and the upload happen once.
    """

    def __init__(self, device="cuda"):
        self.device = device
        self._cache = {}

    def get(self, seq_len: int, block_size: int, *, mask=None, **options):
        """(row_ptr, col_idx, nnz) on the device; ``options`` as for build_pattern."""
        mkey = (None if mask is None else
                np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8).tobytes())
        okey = tuple(sorted((k, tuple(int(g) for g in v) if k == "global_blocks" and v is not None
                             else v) for k, v in options.items()))
        key = (seq_len, block_size, mkey, okey)
        hit = self._cache.get(key)
        if hit is None:
            row_ptr, col_idx = build_pattern(seq_len, block_size, mask=mask, **options)
            hit = (row_ptr.to(self.device, non_blocking=False),
                   col_idx.to(self.device, non_blocking=False), int(col_idx.numel()))
            self._cache[key] = hit
        return hit

    def split_plan(self, seq_len: int, block_size: int, *, mask=None, **options):
        """The device RowSplitPlan of the same pattern, or None when no row is
        long enough to split (cached with the pattern)."""
        row_ptr, _, _ = self.get(seq_len, block_size, mask=mask, **options)
        key = ("split", seq_len, block_size,
               None if mask is None else
               np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8).tobytes(),
               tuple(sorted((k, tuple(v) if isinstance(v, (list, tuple)) else v)
                            for k, v in options.items())))
        if key not in self._cache:
            plan = plan_row_split(row_ptr.cpu())
            self._cache[key] = None if plan is None else plan.to(self.device)
        return self._cache[key]
