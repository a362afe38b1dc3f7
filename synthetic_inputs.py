"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the attention method: it draws random
numbers, builds the structural block masks the workloads are defined by, and
names the workload shapes.  Both the CPU oracle and the HIP library receive
exactly the arrays produced here.

Recipe (stated once, used everywhere):

* Q, K, V: ``g = torch.Generator('cpu').manual_seed(seed)``, then Q, K and V
  are drawn in that order with ``torch.randn(B, H, N, d, generator=g,
  dtype=float32)`` and rounded once (round-to-nearest-even) to the workload's
  dtype.  The oracle upcasts those rounded values exactly.
* Bernoulli block mask: its own generator seeded ``seed + 1``;
  ``torch.bernoulli(torch.full((M, M), p, dtype=float64), generator=g)``, then
  the diagonal block is forced on so that no query block is empty.
* Local+global block mask: blocks within +-radius of the diagonal, the global
  columns in every row, and the global rows dense.
* Decode: q [B, H, d] and the KV caches [B, H, N, d] drawn like Q, K, V (one
  generator seeded ``seed``, in that order); cached lengths uniform on
  [1, N] from a generator seeded ``seed + 2``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    block_size: int
    dtype: str          # "f32" or "bf16"
    pattern: str        # "loglinear", "local_global", "bernoulli"
    description: str

    @property
    def M(self) -> int:
        return self.N // self.block_size

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, 32, "f32", "loglinear",
                     "B=1 H=2 N=256 d=64 block 32 (M=8), log-linear, fp32"),
    "worked_example": Workload("worked_example", 1, 8, 4096, 64, 32, "bf16", "loglinear",
                               "B=1 H=8 N=4096 d=64 block 32 (M=128), log-linear k=1..7, "
                               "globals {0,64,127}, bf16"),
    "local_global": Workload("local_global", 2, 16, 8192, 128, 64, "bf16", "local_global",
                             "B=2 H=16 N=8192 d=128 block 64 (M=128), +-4 blocks + global "
                             "blocks 0 and M-1 (rows 0, M-1 dense), bf16"),
    "random_mask": Workload("random_mask", 128, 8, 2048, 64, 64, "bf16", "bernoulli",
                            "B=128 H=8 N=2048 d=64 block 64 (M=32), Bernoulli(0.3) block mask "
                            "+ diagonal, bf16"),
    "long": Workload("long", 1, 32, 32768, 128, 64, "bf16", "loglinear",
                     "B=1 H=32 N=32768 d=128 block 64 (M=512), log-linear k=1..9, "
                     "globals {0,256,511}, bf16"),
    # Same pattern, block and head size as the worked example with the batch
    # raised until the grid (32768 workgroups) fills the GPU many times over.
    "worked_example_b32": Workload("worked_example_b32", 32, 8, 4096, 64, 32, "bf16", "loglinear",
                                   "B=32 H=8 N=4096 d=64 block 32 (M=128), log-linear, bf16"),
    # Decode: one new token per sequence against a KV cache of capacity N, the
    # cached lengths drawn uniformly from [1, N] (a serving batch's length mix).
    "decode_worked_example": Workload("decode_worked_example", 128, 8, 4096, 64, 32, "bf16",
                                      "loglinear",
                                      "decode, B=128 sequences, H=8, KV cache N=4096 d=64 block "
                                      "32 (M=128), log-linear, lengths U[1, 4096], bf16"),
    "decode_long": Workload("decode_long", 16, 32, 32768, 128, 64, "bf16", "loglinear",
                            "decode, B=16 sequences, H=32, KV cache N=32768 d=128 block 64 "
                            "(M=512), log-linear, lengths U[1, 32768], bf16"),
}

BERNOULLI_KEEP_P = 0.3
LOCAL_GLOBAL_RADIUS = 4


def make_qkv(B: int, H: int, N: int, d: int, dtype=torch.bfloat16, seed: int = 0):
    """Q, K, V as CPU tensors [B, H, N, d] of ``dtype`` (see module recipe)."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def bernoulli_block_mask(M: int, p: float = BERNOULLI_KEEP_P, seed: int = 0,
                         force_diagonal: bool = True) -> np.ndarray:
    """[M, M] uint8 mask; each block kept with probability p, diagonal forced on."""
    g = torch.Generator("cpu").manual_seed(seed + 1)
    draw = torch.bernoulli(torch.full((M, M), p, dtype=torch.float64), generator=g)
    mask = draw.numpy().astype(np.uint8)
    if force_diagonal:
        np.fill_diagonal(mask, 1)
    return mask


def local_global_block_mask(M: int, radius: int = LOCAL_GLOBAL_RADIUS,
                            global_blocks=None) -> np.ndarray:
    """[M, M] uint8 mask: |i - j| <= radius, global columns, global rows dense."""
    if global_blocks is None:
        global_blocks = (0, M - 1)
    i = np.arange(M)[:, None]
    j = np.arange(M)[None, :]
    mask = (np.abs(i - j) <= radius).astype(np.uint8)
    for g in global_blocks:
        mask[:, g] = 1
        mask[g, :] = 1
    return mask


def workload_block_mask(w: Workload, seed: int = 0):
    """The user block mask a workload is defined by, or None for the built-in
    log-linear pattern."""
    if w.pattern == "loglinear":
        return None
    if w.pattern == "local_global":
        return local_global_block_mask(w.M)
    if w.pattern == "bernoulli":
        return bernoulli_block_mask(w.M, seed=seed)
    raise ValueError(w.pattern)


def decode_lengths(B: int, n_cap: int, seed: int = 0) -> torch.Tensor:
    """Cached lengths of B sequences, uniform on [1, n_cap], int32 (CPU);
    their own generator, seeded ``seed + 2``."""
    g = torch.Generator("cpu").manual_seed(seed + 2)
    return torch.randint(1, n_cap + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def make_decode_inputs(B: int, H: int, n_cap: int, d: int, dtype=torch.bfloat16, seed: int = 0):
    """q [B, H, d] and the caches [B, H, n_cap, d]: drawn in the order q, K, V
    with one generator seeded ``seed`` (float32 N(0,1), rounded once)."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, d, generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn(B, H, n_cap, d, generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn(B, H, n_cap, d, generator=g, dtype=torch.float32).to(dtype)
    return q, k, v


def random_block_mask(M: int, p: float, seed: int, force_diagonal: bool = True) -> np.ndarray:
    """Generic Bernoulli mask for small parity cases (numpy generator)."""
    rng = np.random.default_rng(seed)
    mask = (rng.random((M, M)) < p).astype(np.uint8)
    if force_diagonal:
        np.fill_diagonal(mask, 1)
    return mask
